"""Pins for the oracle's forward with radial weights w = h Wr (per-edge radial
features h[E, K] times a shared last-layer matrix Wr[K, P, C]):

  * one basis function with h = 1 is the plain forward with w[e] = Wr[0];
  * the forward is linear in h and in Wr;
  * the weights against an explicit double loop;
  * the VJP (gx, gh, gr, gWr) against central differences of <G, out> in
    x, h, vec and Wr, and the weight gradients against the plain VJP's gw
    contracted by hand for one basis function.
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


@pytest.mark.parametrize("L,K", [(1, 3), (2, 8)])
def test_vjp_finite_differences(L, K):
    wl, h, Wr = case(L, 3, K, 10 + L)
    g = np.random.default_rng(20 + L)
    G = g.standard_normal((wl.n_dst, oracle.dims(L)["Dout"], 3))
    gx, gh, gr, gWr = oracle.vjp_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr, G)

    def f(x=wl.x, hh=h, vec=wl.vec, ww=Wr):
        return (G * oracle.fwd_radial(L, wl.row_ptr, wl.src, vec, x, hh, ww)).sum()

    eps = 1e-6
    x = wl.x.astype(np.float64)
    vec = wl.vec.astype(np.float64)
    for name, arr, grad, kw in (("x", x, gx, "x"), ("h", h, gh, "hh"), ("vec", vec, gr, "vec"),
                                ("Wr", Wr, gWr, "ww")):
        for t in range(4):
            idx = tuple(int(g.integers(s)) for s in arr.shape)
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += eps
            a2[idx] -= eps
            fd = (f(**{kw: a1}) - f(**{kw: a2})) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_weight_gradients_single_basis():
    """K = 1: gh[e] = sum_{p,u} gw[e,p,u] Wr[0,p,u] and gWr[0] = sum_e h[e] gw[e]."""
    wl, h, Wr = case(2, 2, 1, 7)
    G = np.random.default_rng(8).standard_normal((wl.n_dst, oracle.dims(2)["Dout"], 2))
    w = oracle.radial_weights(h, Wr)
    _, gw, _ = oracle.vjp(2, wl.row_ptr, wl.src, wl.vec, wl.x, w, G)
    _, gh, _, gWr = oracle.vjp_radial(2, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr, G)
    for e in range(wl.E):
        assert abs(gh[e, 0] - float((gw[e] * Wr[0]).sum())) < 1e-12
    want = sum(h[e, 0] * gw[e] for e in range(wl.E))
    np.testing.assert_allclose(gWr[0], want, atol=1e-12)


@pytest.mark.parametrize("L,K,cot", [(1, 3, ("x", "h", "r")), (2, 5, ("x", "h", "r")), (2, 2, ("h",)),
                                     (3, 2, ("x", "r"))])
def test_vjp2_radial_finite_differences(L, K, cot):
    """The radial VJP-of-VJP against central differences of
    S = <X', gx> + <H', gh> + <R', gr> (gx, gh, gr from the oracle's radial
    VJP, itself pinned by differences of the forward) in x, h, vec, G and Wr."""
    wl, h, Wr = case(L, 2, K, 40 + L + K)
    g = np.random.default_rng(50 + L + K)
    D = oracle.dims(L)
    G = g.standard_normal((wl.n_dst, D["Dout"], 2))
    Xp = g.standard_normal(wl.x.shape) if "x" in cot else None
    Hp = g.standard_normal(h.shape) if "h" in cot else None
    Rp = g.standard_normal((wl.E, 3)) if "r" in cot else None
    dx, dh, dr, dG, dWr = oracle.vjp2_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr, G, Xp, Hp, Rp)
    x0, vec0 = wl.x.astype(np.float64), wl.vec.astype(np.float64)

    def S(x=x0, hh=h, vec=vec0, GG=G, ww=Wr):
        gx, gh, gr, _ = oracle.vjp_radial(L, wl.row_ptr, wl.src, vec, x, hh, ww, GG)
        t = 0.0
        if Xp is not None:
            t += (Xp * gx).sum()
        if Hp is not None:
            t += (Hp * gh).sum()
        if Rp is not None:
            t += (Rp * gr).sum()
        return t

    eps = 1e-6
    for name, arr, grad, kw in (("x", x0, dx, "x"), ("h", h, dh, "hh"), ("vec", vec0, dr, "vec"),
                                ("G", G, dG, "GG"), ("Wr", Wr, dWr, "ww")):
        for t in range(4):
            idx = tuple(int(g.integers(sz)) for sz in arr.shape)
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += eps
            a2[idx] -= eps
            fd = (S(**{kw: a1}) - S(**{kw: a2})) / (2 * eps)
            assert abs(fd - grad[idx]) < 2e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_vjp2_radial_single_basis_is_plain_vjp2():
    """With one basis function and h = 1 the radial VJP-of-VJP is the plain
    one with w = Wr[0] and W' = H' Wr[0], and dh = sum over paths and
    channels of dw Wr[0]."""
    L, C = 2, 3
    wl, _, Wr = case(L, C, 1, 61)
    g = np.random.default_rng(62)
    h = np.ones((wl.E, 1))
    G = g.standard_normal((wl.n_dst, oracle.dims(L)["Dout"], C))
    Hp = g.standard_normal((wl.E, 1))
    Rp = g.standard_normal((wl.E, 3))
    dx, dh, dr, dG, _ = oracle.vjp2_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr, G, wl.ggx, Hp, Rp)
    w = np.broadcast_to(Wr[0], (wl.E,) + Wr.shape[1:])
    Wp = Hp[:, :, None] * Wr[0][None]
    rdx, rdw, rdr, rdG = oracle.vjp2(L, wl.row_ptr, wl.src, wl.vec, wl.x, w, G, wl.ggx, Wp, Rp)
    np.testing.assert_allclose(dx, rdx, atol=1e-12)
    np.testing.assert_allclose(dr, rdr, atol=1e-12)
    np.testing.assert_allclose(dG, rdG, atol=1e-12)
    np.testing.assert_allclose(dh[:, 0], (rdw * Wr[0][None]).sum(axis=(1, 2)), atol=1e-12)
