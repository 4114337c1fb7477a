"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: hand-worked
fixtures under tests/golden/, closed forms, brute-force loops written here in
plain Python, special cases that reduce to textbook or library routines, and
structural invariants. Page tags follow the oracle's header:
[KR] "RetNet - Retentive Network - A Successor to Transformer for LLMs",
[JP] the jisaku.com RetNet glossary entry, [EN] "What Is RetNet ? could it
challenge the dominance of the Transformer ?".
"""

import os

import numpy as np
import pytest
import torch

from oracle import retention_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tol(ref):
    # fp64 agreement between the oracle's own forms: 1e-10 * max(1, max|o|).
    return 1e-10 * max(1.0, float(np.max(np.abs(ref))))


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _inputs(B, H, N, dk, dv, seed):
    q = _rand((B, H, N, dk), seed)
    k = _rand((B, H, N, dk), seed + 1)
    v = _rand((B, H, N, dv), seed + 2)
    return q, k, v


def _gammas(H):
    return np.array([1.0 - 2.0 ** (-5 - h) for h in range(H)])


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((parts[0], [float(x) for x in parts[1:]]))
    return rows


# --------------------------------------------------------------------------
# Hand-worked fixtures
# --------------------------------------------------------------------------


def test_golden_recurrent_hand_example():
    """[KR] Key Equations, recurrent form, worked by hand (tests/golden)."""
    rows = _read_fixture("recurrent_hand_example.txt")
    gamma = [r[1][0] for r in rows if r[0] == "gamma"][0]
    get = lambda tag: {int(r[1][0]): r[1][1:] for r in rows if r[0] == tag}
    qd, kd, vd, od, Sd = get("q"), get("k"), get("v"), get("o"), get("S")
    N = len(qd)
    q = np.array([qd[n] for n in range(N)])[None, None]
    k = np.array([kd[n] for n in range(N)])[None, None]
    v = np.array([vd[n] for n in range(N)])[None, None]
    o_ref = np.array([od[n] for n in range(N)])
    S_ref = np.array([Sd[i] for i in range(len(Sd))])
    g = np.array([gamma])

    o_rec, S_rec = orc.recurrent(q, k, v, g)
    np.testing.assert_allclose(o_rec[0, 0], o_ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(S_rec[0, 0], S_ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.parallel(q, k, v, g)[0, 0], o_ref, rtol=0, atol=1e-15)
    for C in (1, 2, 5):
        o_ch, S_ch = orc.chunkwise(q, k, v, g, C)
        np.testing.assert_allclose(o_ch[0, 0], o_ref, rtol=0, atol=1e-15)
        np.testing.assert_allclose(S_ch[0, 0], S_ref, rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.state_after(k, v, g)[0, 0], S_ref, rtol=0, atol=1e-15)


def test_golden_geometric_series():
    """d = 1, all-ones inputs: o_n is a geometric series (tests/golden)."""
    for tag, vals in _read_fixture("geometric_series.txt"):
        assert tag == "series"
        gamma, expect = vals[0], np.array(vals[1:])
        N = len(expect)
        ones = np.ones((1, 1, N, 1))
        g = np.array([gamma])
        np.testing.assert_allclose(orc.parallel(ones, ones, ones, g)[0, 0, :, 0], expect, rtol=0, atol=1e-15)
        np.testing.assert_allclose(orc.recurrent(ones, ones, ones, g)[0][0, 0, :, 0], expect, rtol=0, atol=1e-15)
        for C in (1, 2, 3):
            np.testing.assert_allclose(orc.chunkwise(ones, ones, ones, g, C)[0][0, 0, :, 0], expect, rtol=0, atol=1e-15)


@pytest.mark.parametrize("gamma", [1 - 2.0 ** -5, 1 - 2.0 ** -8, 1 - 2.0 ** -12, 0.5])
def test_closed_form_all_ones(gamma):
    """o_n = (1 - gamma^(n+1)) / (1 - gamma) for d = 1, all-ones q, k, v, N = 64."""
    N = 64
    ones = np.ones((1, 1, N, 1))
    g = np.array([gamma])
    n = np.arange(N)
    expect = (1.0 - gamma ** (n + 1)) / (1.0 - gamma)
    tol = 1e-12 * expect.max()
    np.testing.assert_allclose(orc.parallel(ones, ones, ones, g)[0, 0, :, 0], expect, rtol=0, atol=tol)
    np.testing.assert_allclose(orc.recurrent(ones, ones, ones, g)[0][0, 0, :, 0], expect, rtol=0, atol=tol)
    np.testing.assert_allclose(orc.chunkwise(ones, ones, ones, g, 16)[0][0, 0, :, 0], expect, rtol=0, atol=tol)


def test_golden_groupnorm_hand_example():
    """Per-head GroupNorm of one row, worked by hand (tests/golden)."""
    d = dict(_read_fixture("groupnorm_hand_example.txt"))
    o = np.array(d["row"])[None, None, None, :]
    np.testing.assert_allclose(orc.group_norm(o, eps=0.0)[0, 0, 0], d["y"], rtol=0, atol=1e-14)
    y = orc.group_norm(o, eps=0.0, weight=np.array(d["weight"]), bias=np.array(d["bias"]))
    np.testing.assert_allclose(y[0, 0, 0], d["y_affine"], rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# Brute force in plain Python loops
# --------------------------------------------------------------------------


def _brute_parallel(q, k, v, gamma):
    """Literal double loop over (n, m), scalar arithmetic only."""
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    out = [[[[0.0] * dv for _ in range(N)] for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            g = float(gamma[h])
            for n in range(N):
                for m in range(n + 1):
                    s = 0.0
                    for c in range(dk):
                        s += float(q[b, h, n, c]) * float(k[b, h, m, c])
                    w = s * g ** (n - m)
                    for c in range(dv):
                        out[b][h][n][c] += w * float(v[b, h, m, c])
    return np.array(out)


def _brute_state_one_based(k, v, gamma):
    """S_N = sum_{m=1..N} gamma^(N-m) k_m^T v_m with 1-based m, as stated for the state check."""
    B, H, N, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            g = float(gamma[h])
            for m1 in range(1, N + 1):
                w = g ** (N - m1)
                for i in range(dk):
                    for j in range(dv):
                        S[b, h, i, j] += w * float(k[b, h, m1 - 1, i]) * float(v[b, h, m1 - 1, j])
    return S


@pytest.mark.parametrize("N,dk,dv,H", [(1, 1, 1, 1), (5, 2, 3, 2), (12, 3, 2, 3), (9, 4, 4, 1)])
def test_brute_force_outputs(N, dk, dv, H):
    q, k, v = _inputs(2, H, N, dk, dv, seed=10 * N + dk)
    g = np.array([0.9, 0.6, 0.3])[:H]
    ref = _brute_parallel(q, k, v, g)
    tol = _tol(ref)
    np.testing.assert_allclose(orc.parallel(q, k, v, g), ref, rtol=0, atol=tol)
    np.testing.assert_allclose(orc.recurrent(q, k, v, g)[0], ref, rtol=0, atol=tol)
    for C in (1, 2, 4, 7, N + 3):
        np.testing.assert_allclose(orc.chunkwise(q, k, v, g, C)[0], ref, rtol=0, atol=tol)
    rows = [0, N // 2, N - 1]
    np.testing.assert_allclose(orc.parallel_rows(q, k, v, g, rows), ref[:, :, rows], rtol=0, atol=tol)


@pytest.mark.parametrize("N", [1, 3, 11])
def test_brute_force_state(N):
    q, k, v = _inputs(1, 2, N, 3, 2, seed=N)
    g = np.array([0.8, 0.35])
    ref = _brute_state_one_based(k, v, g)
    tol = _tol(ref)
    np.testing.assert_allclose(orc.recurrent(q, k, v, g)[1], ref, rtol=0, atol=tol)
    np.testing.assert_allclose(orc.state_after(k, v, g), ref, rtol=0, atol=tol)
    for C in (1, 2, 4, N + 1):
        np.testing.assert_allclose(orc.chunkwise(q, k, v, g, C)[1], ref, rtol=0, atol=tol)


# --------------------------------------------------------------------------
# The three forms agree (claimed exact by the pages) on random inputs
# --------------------------------------------------------------------------


@pytest.mark.parametrize(
    "B,H,N,dk,dv,C,with_state",
    [
        (1, 1, 64, 16, 16, 16, False),  # the single-head fp32 case
        (1, 1, 61, 16, 16, 16, False),  # ragged last chunk
        (2, 4, 61, 8, 12, 16, True),    # multi-head gamma_h, dk != dv, starting state
        (1, 3, 40, 5, 7, 9, True),
    ],
)
def test_three_forms_agree(B, H, N, dk, dv, C, with_state):
    q, k, v = _inputs(B, H, N, dk, dv, seed=N + C)
    g = _gammas(H)
    S0 = _rand((B, H, dk, dv), seed=99) if with_state else None
    o_par = orc.parallel(q, k, v, g, state_in=S0)
    o_rec, S_rec = orc.recurrent(q, k, v, g, state_in=S0)
    o_chk, S_chk = orc.chunkwise(q, k, v, g, C, state_in=S0)
    tol = _tol(o_rec)
    assert np.max(np.abs(o_par - o_rec)) <= tol
    assert np.max(np.abs(o_chk - o_rec)) <= tol
    assert np.max(np.abs(S_chk - S_rec)) <= _tol(S_rec)
    assert np.max(np.abs(orc.state_after(k, v, g, S0) - S_rec)) <= _tol(S_rec)


# --------------------------------------------------------------------------
# Special cases that reduce to textbook routines
# --------------------------------------------------------------------------


def test_gamma_one_is_causal_linear_attention():
    """gamma = 1: O = tril(Q K^T) V, causal linear attention (numpy.tril)."""
    q, k, v = _inputs(1, 1, 20, 4, 3, seed=5)
    ref = np.tril(q[0, 0] @ k[0, 0].T) @ v[0, 0]
    g = np.array([1.0])
    tol = _tol(ref)
    np.testing.assert_allclose(orc.parallel(q, k, v, g)[0, 0], ref, rtol=0, atol=tol)
    np.testing.assert_allclose(orc.recurrent(q, k, v, g)[0][0, 0], ref, rtol=0, atol=tol)
    np.testing.assert_allclose(orc.chunkwise(q, k, v, g, 6)[0][0, 0], ref, rtol=0, atol=tol)


def test_gamma_zero_keeps_only_the_diagonal():
    """gamma = 0: o_n = (q_n . k_n) v_n."""
    q, k, v = _inputs(1, 1, 10, 3, 2, seed=6)
    ref = np.einsum("nk,nk->n", q[0, 0], k[0, 0])[:, None] * v[0, 0]
    g = np.array([0.0])
    np.testing.assert_allclose(orc.parallel(q, k, v, g)[0, 0], ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(orc.recurrent(q, k, v, g)[0][0, 0], ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(orc.chunkwise(q, k, v, g, 4)[0][0, 0], ref, rtol=0, atol=1e-13)


def test_decay_mask_is_lower_triangular_powers():
    D = orc.decay_mask(4, 0.5)
    expect = np.array(
        [[1, 0, 0, 0], [0.5, 1, 0, 0], [0.25, 0.5, 1, 0], [0.125, 0.25, 0.5, 1]], dtype=np.float64
    )
    np.testing.assert_array_equal(D, expect)


def test_state_readout_closed_form():
    """k = 0, q = 1, d = 1: only the starting state is read, o_n = gamma^(n+1) s."""
    N, s, gamma = 13, 3.0, 0.7
    q = np.ones((1, 1, N, 1))
    k = np.zeros((1, 1, N, 1))
    v = _rand((1, 1, N, 1), seed=3)
    S0 = np.full((1, 1, 1, 1), s)
    g = np.array([gamma])
    expect = s * gamma ** (np.arange(N) + 1.0)
    np.testing.assert_allclose(orc.recurrent(q, k, v, g, S0)[0][0, 0, :, 0], expect, rtol=1e-14)
    np.testing.assert_allclose(orc.parallel(q, k, v, g, S0)[0, 0, :, 0], expect, rtol=1e-14)
    for C in (1, 4, 5, 20):
        o, S = orc.chunkwise(q, k, v, g, C, S0)
        np.testing.assert_allclose(o[0, 0, :, 0], expect, rtol=1e-14)
        np.testing.assert_allclose(S[0, 0, 0, 0], s * gamma ** N, rtol=1e-14)


def test_chunk_one_is_recurrent_and_chunk_n_is_parallel():
    q, k, v = _inputs(1, 2, 17, 3, 5, seed=8)
    g = _gammas(2)
    o_rec, S_rec = orc.recurrent(q, k, v, g)
    o1, S1 = orc.chunkwise(q, k, v, g, 1)
    assert np.max(np.abs(o1 - o_rec)) <= _tol(o_rec)
    assert np.max(np.abs(S1 - S_rec)) <= _tol(S_rec)
    oN, _ = orc.chunkwise(q, k, v, g, 17)
    assert np.max(np.abs(oN - orc.parallel(q, k, v, g))) <= _tol(o_rec)


# --------------------------------------------------------------------------
# Structure
# --------------------------------------------------------------------------


def test_split_sequence_seam():
    """Prefill then continue from the carried state equals one pass."""
    q, k, v = _inputs(2, 3, 50, 4, 6, seed=12)
    g = _gammas(3)
    o_all, S_all = orc.chunkwise(q, k, v, g, 8)
    N1 = 21
    o_a, S_a = orc.chunkwise(q[:, :, :N1], k[:, :, :N1], v[:, :, :N1], g, 8)
    o_b, S_b = orc.chunkwise(q[:, :, N1:], k[:, :, N1:], v[:, :, N1:], g, 8, state_in=S_a)
    np.testing.assert_allclose(np.concatenate([o_a, o_b], axis=2), o_all, rtol=0, atol=_tol(o_all))
    np.testing.assert_allclose(S_b, S_all, rtol=0, atol=_tol(S_all))


def test_linearity_in_v():
    q, k, v1 = _inputs(1, 2, 19, 3, 4, seed=20)
    v2 = _rand(v1.shape, seed=21)
    g = _gammas(2)
    a, b = 0.7, -1.3
    lhs = orc.chunkwise(q, k, a * v1 + b * v2, g, 5)[0]
    rhs = a * orc.chunkwise(q, k, v1, g, 5)[0] + b * orc.chunkwise(q, k, v2, g, 5)[0]
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=_tol(lhs))


def test_head_independence():
    """A multi-scale head equals a single-head run with that head's gamma."""
    q, k, v = _inputs(1, 4, 15, 3, 3, seed=30)
    g = _gammas(4)
    o = orc.parallel(q, k, v, g)
    for h in range(4):
        single = orc.parallel(q[:, h : h + 1], k[:, h : h + 1], v[:, h : h + 1], g[h : h + 1])
        np.testing.assert_allclose(o[:, h : h + 1], single, rtol=0, atol=_tol(o))


def test_causality():
    q, k, v = _inputs(1, 1, 24, 3, 3, seed=40)
    g = np.array([0.9])
    o = orc.chunkwise(q, k, v, g, 5)[0]
    t = 13
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, :, t] += 5.0
    k2[:, :, t] -= 2.0
    v2[:, :, t] *= -3.0
    o2 = orc.chunkwise(q2, k2, v2, g, 5)[0]
    np.testing.assert_array_equal(o[:, :, :t], o2[:, :, :t])
    assert np.max(np.abs(o[:, :, t:] - o2[:, :, t:])) > 1e-3


def test_step_matches_recurrence():
    q, k, v = _inputs(2, 3, 6, 4, 5, seed=50)
    g = _gammas(3)
    S = _rand((2, 3, 4, 5), seed=51)
    o_ref, S_ref = orc.recurrent(q, k, v, g, S)
    for n in range(6):
        o_n, S = orc.recurrent_step(q[:, :, n], k[:, :, n], v[:, :, n], g, S)
        np.testing.assert_allclose(o_n, o_ref[:, :, n], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# GroupNorm
# --------------------------------------------------------------------------


def test_group_norm_matches_torch_group_norm():
    """Per-head GN over dv equals torch.nn.functional.group_norm with H groups."""
    B, H, N, dv = 2, 3, 7, 8
    o = _rand((B, H, N, dv), seed=60, std=3.0) + 1.5
    w = _rand((H * dv,), seed=61)
    bvec = _rand((H * dv,), seed=62)
    ours = orc.group_norm(o, eps=1e-5, weight=w, bias=bvec)
    # torch layout: (batch*tokens, channels = H*dv), groups = H
    x = torch.from_numpy(o).permute(0, 2, 1, 3).reshape(B * N, H * dv)
    ref = torch.nn.functional.group_norm(x, H, torch.from_numpy(w), torch.from_numpy(bvec), eps=1e-5)
    ref = ref.reshape(B, N, H, dv).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def test_group_norm_invariants():
    o = _rand((1, 2, 5, 16), seed=70, std=2.0)
    eps = 1e-5
    y = orc.group_norm(o, eps=eps)
    var = o.var(axis=-1)
    np.testing.assert_allclose(y.mean(axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=-1), var / (var + eps), rtol=1e-12)
    scale = np.array([3.0, 0.25])[None, :, None, None]
    y2 = orc.group_norm(o * scale, eps=0.0)
    np.testing.assert_allclose(y2, orc.group_norm(o, eps=0.0), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Gated epilogue: swish(gate) * GroupNorm(o)
# --------------------------------------------------------------------------


def _swish_by_tanh(x):
    # sigmoid(x) = (1 + tanh(x / 2)) / 2, an identity independent of the
    # exp-based form the oracle uses.
    return x * 0.5 * (1.0 + np.tanh(0.5 * x))


def test_swish_values_and_identities():
    # sigmoid(1) = e / (1 + e); swish(0) = 0.
    assert orc.swish(np.array([1.0]))[0] == pytest.approx(np.e / (1.0 + np.e), rel=1e-15)
    assert orc.swish(np.array([0.0]))[0] == 0.0
    x = _rand((4000,), seed=80, std=6.0)
    # (the tanh form cancels for very negative x, hence the absolute floor)
    np.testing.assert_allclose(orc.swish(x), _swish_by_tanh(x), rtol=1e-13, atol=1e-14)
    # sigmoid(-x) = 1 - sigmoid(x)  =>  swish(-x) = swish(x) - x
    np.testing.assert_allclose(orc.swish(-x), orc.swish(x) - x, rtol=0, atol=1e-12)
    # limits: identity far right, zero far left, no overflow
    big = np.array([50.0, 700.0, 1e4])
    np.testing.assert_allclose(orc.swish(big), big, rtol=1e-15)
    assert np.all(np.abs(orc.swish(-big)) < 1e-15)


def test_swish_matches_torch_silu():
    x = _rand((1000,), seed=81, std=4.0)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(orc.swish(x), ref, rtol=1e-14, atol=1e-300)


def test_gated_group_norm_special_cases():
    B, H, N, dv = 1, 2, 5, 16
    o = _rand((B, H, N, dv), seed=82, std=2.0) + 0.5
    w = _rand((H * dv,), seed=83)
    bvec = _rand((H * dv,), seed=84)
    y = orc.group_norm(o, 1e-5, w, bvec)
    # a zero gate closes the branch
    np.testing.assert_array_equal(orc.gated_group_norm(o, np.zeros_like(o), 1e-5, w, bvec), 0.0)
    # a large positive gate passes gate * GN(o) (swish(g) = g up to e^-g)
    g = np.full_like(o, 40.0)
    np.testing.assert_allclose(orc.gated_group_norm(o, g, 1e-5, w, bvec), 40.0 * y, rtol=1e-15)
    # elementwise: against the library's silu and group_norm
    gate = _rand((B, H, N, dv), seed=85, std=2.0)
    x = torch.from_numpy(o).permute(0, 2, 1, 3).reshape(B * N, H * dv)
    gn = torch.nn.functional.group_norm(x, H, torch.from_numpy(w), torch.from_numpy(bvec), eps=1e-5)
    gt = torch.from_numpy(gate).permute(0, 2, 1, 3).reshape(B * N, H * dv)
    ref = (torch.nn.functional.silu(gt) * gn).reshape(B, N, H, dv).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(orc.gated_group_norm(o, gate, 1e-5, w, bvec), ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Backward: gradients of O and of the final state
# --------------------------------------------------------------------------


def _loss(q, k, v, S0, gamma, W, U):
    """L = sum(W * O) + sum(U * S_N) through the oracle's (pinned) forward maps."""
    return float(np.sum(W * orc.parallel(q, k, v, gamma, state_in=S0))
                 + np.sum(U * orc.state_after(k, v, gamma, state_in=S0)))


def test_backward_matches_finite_differences():
    B, H, N, dk, dv = 1, 2, 6, 3, 4
    q, k, v = _inputs(B, H, N, dk, dv, seed=90)
    S0 = _rand((B, H, dk, dv), seed=91)
    W = _rand((B, H, N, dv), seed=92)
    U = _rand((B, H, dk, dv), seed=93)
    g = np.array([0.9, 0.55])
    grads = orc.backward(q, k, v, g, W, state_in=S0, d_state_out=U)
    eps = 1e-6
    for x, gx in zip((q, k, v, S0), grads):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = [q, k, v, S0]
            i = next(j for j, a in enumerate(args) if a is x)
            args_p, args_m = list(args), list(args)
            args_p[i], args_m[i] = xp, xm
            fd[idx] = (_loss(*args_p, g, W, U) - _loss(*args_m, g, W, U)) / (2 * eps)
        np.testing.assert_allclose(gx, fd, rtol=0, atol=1e-7)


def test_backward_matches_torch_autograd_of_the_recurrence():
    """Autograd through the token-by-token recurrence (update, then read out)."""
    B, H, N, dk, dv = 2, 2, 9, 4, 3
    q, k, v = _inputs(B, H, N, dk, dv, seed=94)
    S0 = _rand((B, H, dk, dv), seed=95)
    W = _rand((B, H, N, dv), seed=96)
    U = _rand((B, H, dk, dv), seed=97)
    g = np.array([0.8, 0.3])
    tq, tk, tv, tS = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v, S0))
    gam = torch.tensor(g, dtype=torch.float64)[None, :, None, None]
    S = tS
    outs = []
    for n in range(N):
        S = gam * S + tk[:, :, n, :, None] * tv[:, :, n, None, :]
        outs.append(torch.einsum("bhk,bhkv->bhv", tq[:, :, n], S))
    O = torch.stack(outs, dim=2)
    L = (O * torch.from_numpy(W)).sum() + (S * torch.from_numpy(U)).sum()
    L.backward()
    ours = orc.backward(q, k, v, g, W, state_in=S0, d_state_out=U)
    for got, ref in zip(ours, (tq.grad, tk.grad, tv.grad, tS.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-11)


def test_backward_without_state_terms():
    """No S0 and no dS_N: dS0 is None, and the gradients equal those with zero tensors."""
    q, k, v = _inputs(1, 1, 7, 3, 5, seed=98)
    W = _rand((1, 1, 7, 5), seed=99)
    g = np.array([0.7])
    a = orc.backward(q, k, v, g, W)
    b = orc.backward(q, k, v, g, W, state_in=np.zeros((1, 1, 3, 5)), d_state_out=np.zeros((1, 1, 3, 5)))
    assert a[3] is None
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_allclose(x, y, rtol=0, atol=0)
    np.testing.assert_allclose(b[3], orc.backward(q, k, v, g, W, state_in=np.zeros((1, 1, 3, 5)))[3], atol=0)


def test_backward_rows_equal_backward():
    """The per-row gradients equal the matrix form's rows (first, last, middle)."""
    q, k, v = _inputs(2, 2, 13, 3, 4, seed=100)
    S0 = _rand((2, 2, 3, 4), seed=101)
    W = _rand((2, 2, 13, 4), seed=102)
    U = _rand((2, 2, 3, 4), seed=103)
    g = np.array([0.85, 0.4])
    full = orc.backward(q, k, v, g, W, state_in=S0, d_state_out=U)
    rows = [0, 5, 12]
    part = orc.backward_rows(q, k, v, g, W, rows, state_in=S0, d_state_out=U)
    for a, b in zip(part, full[:3]):
        np.testing.assert_allclose(a, b[:, :, rows], rtol=0, atol=1e-12)
