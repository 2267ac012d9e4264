"""Pins for the oracle's forward with radial weights w = h Wr (per-edge radial
features h[E, K] times a shared last-layer matrix Wr[K, P, C]):

  * one basis function with h = 1 is the plain forward with w[e] = Wr[0];
  * the forward is linear in h and in Wr;
  * the weights against an explicit double loop.
"""
import numpy as np
import pytest

import oracle
import workloads


def case(L, C, K, seed):
    wl = workloads.small(L, C, 9, 5, seed=seed)
    g = np.random.default_rng(seed)
    P = len(oracle.paths(L))
    h = g.standard_normal((wl.E, K))
    Wr = g.standard_normal((K, P, C)) / np.sqrt(P * K)
    return wl, h, Wr


def test_single_basis_is_plain_forward():
    wl, _, Wr = case(2, 3, 1, 1)
    h = np.ones((wl.E, 1))
    got = oracle.fwd_radial(2, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr)
    want = oracle.fwd(2, wl.row_ptr, wl.src, wl.vec, wl.x, np.broadcast_to(Wr[0], (wl.E,) + Wr.shape[1:]))
    np.testing.assert_allclose(got, want, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2])
def test_linear_in_h_and_Wr(L):
    wl, h, Wr = case(L, 2, 4, 2 + L)
    g = np.random.default_rng(9)
    h2, Wr2 = g.standard_normal(h.shape), g.standard_normal(Wr.shape)
    f = lambda hh, ww: oracle.fwd_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, hh, ww)
    np.testing.assert_allclose(f(h + 2 * h2, Wr), f(h, Wr) + 2 * f(h2, Wr), atol=1e-11)
    np.testing.assert_allclose(f(h, Wr - 3 * Wr2), f(h, Wr) - 3 * f(h, Wr2), atol=1e-11)


def test_weights_against_loops():
    g = np.random.default_rng(3)
    h = g.standard_normal((5, 3))
    Wr = g.standard_normal((3, 4, 2))
    w = oracle.radial_weights(h, Wr)
    for e in range(5):
        for p in range(4):
            for u in range(2):
                assert abs(w[e, p, u] - sum(h[e, k] * Wr[k, p, u] for k in range(3))) < 1e-12
