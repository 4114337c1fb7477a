"""Pins of the oracle's xPos rotation (oracle.retention_oracle.xpos_rotate).

The pages name a complex rotation of Q and K by position ("RetNet - Retentive
Network - A Successor to Transformer for LLMs", Key components, 3. xPos) and
a conjugate in the retention product ("RetNet入門", the parallel
representation), with no formula or angle schedule. The rotation for given
angles theta is pinned here by what the mathematics fixes:
  * a hand-worked fixture (quarter and half turns, tests/golden);
  * complex multiplication done by numpy's complex128 arithmetic;
  * lengths of the feature pairs are preserved; zero angles and position 0
    leave the input unchanged; rotations compose (positions add);
  * the rotated scores depend on positions only through n - m (shifting
    every position leaves q'.k' and the whole retention output unchanged),
    and equal Re(sum_i zq_i conj(zk_i) exp(i (n - m) theta_i)).
Mutants (a reversed turn, the two halves of d paired instead of neighbours,
positions counted from 1) are planted in copies here and each is caught.
The angle schedule itself (which theta a caller passes) is not fixed by the
pages: parity unpinned for any particular schedule.
"""

import numpy as np
import pytest

from oracle import retention_oracle as orc
from tests.test_oracle import _gammas, _inputs, _rand, _read_fixture


def _theta(d, seed=5):
    rng = np.random.default_rng(seed)
    return rng.uniform(0.0, 3.0, d // 2)


def test_golden_quarter_turns():
    rows = _read_fixture("xpos_quarter_turns.txt")
    theta = [r[1] for r in rows if r[0] == "theta"][0]
    x = np.array([r[1][1:] for r in rows if r[0] == "x"])
    y = np.array([r[1][1:] for r in rows if r[0] == "y"])
    np.testing.assert_allclose(orc.xpos_rotate(x, theta), y, rtol=0, atol=1e-15)
    x5 = [r[1] for r in rows if r[0] == "x5"][0]
    y5 = [r[1] for r in rows if r[0] == "y5"][0]
    got = orc.xpos_rotate(np.array([x5[1:]]), theta, pos0=int(x5[0]))
    np.testing.assert_allclose(got[0], y5[1:], rtol=0, atol=1e-14)


def test_matches_complex_multiplication():
    x = _rand((2, 3, 9, 8), 11)
    theta = _theta(8)
    pos0 = 1234
    z = x[..., 0::2] + 1j * x[..., 1::2]
    n = pos0 + np.arange(9)
    zr = z * np.exp(1j * n[:, None] * theta[None, :])
    y = orc.xpos_rotate(x, theta, pos0)
    np.testing.assert_allclose(y[..., 0::2], zr.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[..., 1::2], zr.imag, rtol=0, atol=1e-12)


def test_pair_lengths_identity_and_composition():
    x = _rand((1, 2, 7, 6), 12)
    theta = _theta(6, seed=6)
    y = orc.xpos_rotate(x, theta, pos0=3)
    np.testing.assert_allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.hypot(x[..., 0::2], x[..., 1::2]),
                               rtol=1e-13)
    np.testing.assert_array_equal(orc.xpos_rotate(x, np.zeros(3), pos0=99), x)
    np.testing.assert_allclose(orc.xpos_rotate(x, theta)[..., 0, :], x[..., 0, :], rtol=0, atol=0)
    # A token rotated to position a, then by b more, sits at position a + b.
    t = x[..., 2:3, :]
    np.testing.assert_allclose(orc.xpos_rotate(orc.xpos_rotate(t, theta, pos0=40), theta, pos0=17),
                               orc.xpos_rotate(t, theta, pos0=57), rtol=0, atol=1e-12)


def test_scores_depend_on_relative_position_only():
    q = _rand((1, 1, 6, 8), 13)
    k = _rand((1, 1, 6, 8), 14)
    theta = _theta(8, seed=7)
    s0 = orc.xpos_rotate(q, theta, 0)[0, 0] @ orc.xpos_rotate(k, theta, 0)[0, 0].T
    s1 = orc.xpos_rotate(q, theta, 1000)[0, 0] @ orc.xpos_rotate(k, theta, 1000)[0, 0].T
    np.testing.assert_allclose(s1, s0, rtol=0, atol=1e-11)
    zq = q[0, 0, :, 0::2] + 1j * q[0, 0, :, 1::2]
    zk = k[0, 0, :, 0::2] + 1j * k[0, 0, :, 1::2]
    n = np.arange(6)
    ref = np.real(np.einsum("ni,mi,nmi->nm", zq, np.conj(zk), np.exp(1j * (n[:, None, None] - n[None, :, None])
                                                                       * theta[None, None, :])))
    np.testing.assert_allclose(s0, ref, rtol=0, atol=1e-12)


def test_rotated_retention_is_shift_invariant():
    """With Q and K rotated, the retention output depends only on relative
    positions: every form gives the same output at any starting position."""
    q, k, v = _inputs(1, 2, 10, 6, 4, seed=15)
    g = _gammas(2)
    theta = _theta(6, seed=8)
    ref = orc.parallel(orc.xpos_rotate(q, theta), orc.xpos_rotate(k, theta), v, g)
    qs, ks = orc.xpos_rotate(q, theta, 777), orc.xpos_rotate(k, theta, 777)
    np.testing.assert_allclose(orc.parallel(qs, ks, v, g), ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(orc.recurrent(qs, ks, v, g)[0], ref, rtol=0, atol=1e-11)
    np.testing.assert_allclose(orc.chunkwise(qs, ks, v, g, 4)[0], ref, rtol=0, atol=1e-11)


def _mutant(x, theta, pos0, kind):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    n = pos0 + np.arange(x.shape[-2], dtype=np.float64)
    if kind == "one_based":
        n = n + 1
    ang = n[:, None] * np.asarray(theta)[None, :]
    if kind == "reversed":
        ang = -ang
    c, s = np.cos(ang), np.sin(ang)
    if kind == "halves":
        re, im = x[..., : d // 2], x[..., d // 2:]
    else:
        re, im = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    if kind == "halves":
        y[..., : d // 2], y[..., d // 2:] = re * c - im * s, re * s + im * c
    else:
        y[..., 0::2], y[..., 1::2] = re * c - im * s, re * s + im * c
    return y


@pytest.mark.parametrize("kind", ["reversed", "halves", "one_based"])
def test_mutants_are_caught(kind):
    rows = _read_fixture("xpos_quarter_turns.txt")
    theta = [r[1] for r in rows if r[0] == "theta"][0]
    x = np.array([r[1][1:] for r in rows if r[0] == "x"])
    y = np.array([r[1][1:] for r in rows if r[0] == "y"])
    assert np.max(np.abs(_mutant(x, theta, 0, kind) - y)) > 0.5
    # The unmutated copy reproduces the oracle (the mutant helper itself is sound).
    xr = _rand((1, 1, 5, 8), 16)
    th = _theta(8, seed=9)
    np.testing.assert_allclose(_mutant(xr, th, 3, "none"), orc.xpos_rotate(xr, th, 3), rtol=0, atol=1e-14)


def test_rejects_odd_width_or_wrong_theta():
    with pytest.raises(ValueError):
        orc.xpos_rotate(np.zeros((3, 5)), np.zeros(2))
    with pytest.raises(ValueError):
        orc.xpos_rotate(np.zeros((3, 4)), np.zeros(3))
