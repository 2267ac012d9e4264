"""Pins for the oracle's edge-local tensor product (the convolution's message
per edge, no destination sum):

  * brute force: a dense einsum whose CG comes from sympy and whose SH come
    from scipy, edge by edge;
  * the convolution is the destination sum of the edge-local outputs with
    V_e = x[src_e], and its VJP is the matching source sum of the edge-local
    gV (gw and gr equal edge by edge);
  * the VJP against central differences of <G, out>.
"""
import numpy as np
import pytest

import oracle
import workloads
from test_oracle_conv import _library_dense_cg, _library_sh


def case(L, E, C, seed):
    g = np.random.default_rng(seed)
    vec = workloads.random_vectors(E, 0.8, 5.0, seed).astype(np.float64)
    V = g.standard_normal((E, (L + 1) ** 2, C))
    P = len(oracle.paths(L))
    w = g.standard_normal((E, P, C)) / np.sqrt(P)
    return vec, V, w


@pytest.mark.parametrize("L", [1, 2, 3])
def test_edge_tp_brute_force(L):
    vec, V, w = case(L, 9, 3, L)
    out = oracle.edge_tp_fwd(L, vec, V, w)
    Y = _library_sh(L, vec)
    off = 0
    for p, (l1, l2, l3) in enumerate(oracle.paths(L)):
        T = _library_dense_cg(int(l1), int(l2), int(l3))
        want = np.einsum("abc,eb,eau,eu->ecu", T, Y[:, l2 * l2:(l2 + 1) ** 2], V[:, l1 * l1:(l1 + 1) ** 2], w[:, p])
        np.testing.assert_allclose(out[:, off:off + 2 * l3 + 1], want, atol=1e-12)
        off += 2 * l3 + 1


@pytest.mark.parametrize("L", [1, 2])
def test_conv_is_destination_sum_of_edge_tp(L):
    wl = workloads.small(L, 3, 11, 6, seed=5)
    x, w = wl.x.astype(np.float64), wl.w.astype(np.float64)
    dst = np.repeat(np.arange(wl.n_dst), np.diff(wl.row_ptr))
    per_edge = oracle.edge_tp_fwd(L, wl.vec, x[wl.src], w)
    conv = oracle.fwd(L, wl.row_ptr, wl.src, wl.vec, x, w)
    want = np.zeros_like(conv)
    np.add.at(want, dst, per_edge)
    np.testing.assert_allclose(conv, want, atol=1e-12)
    G = wl.G.astype(np.float64)
    gV, gw_e, gr_e = oracle.edge_tp_vjp(L, wl.vec, x[wl.src], w, G[dst])
    gx, gw, gr = oracle.vjp(L, wl.row_ptr, wl.src, wl.vec, x, w, G)
    want_gx = np.zeros_like(gx)
    np.add.at(want_gx, wl.src, gV)
    np.testing.assert_allclose(gx, want_gx, atol=1e-12)
    np.testing.assert_allclose(gw, gw_e, atol=1e-12)
    np.testing.assert_allclose(gr, gr_e, atol=1e-12)


def test_edge_tp_vjp_finite_differences():
    L = 2
    vec, V, w = case(L, 5, 2, 7)
    G = np.random.default_rng(8).standard_normal(oracle.edge_tp_fwd(L, vec, V, w).shape)
    gV, gw, gr = oracle.edge_tp_vjp(L, vec, V, w, G)
    h = 1e-6

    def S(vec_=vec, V_=V, w_=w):
        return float((G * oracle.edge_tp_fwd(L, vec_, V_, w_)).sum())

    for e in range(5):
        for c in range(3):
            d = np.zeros_like(vec)
            d[e, c] = h
            fd = (S(vec_=vec + d) - S(vec_=vec - d)) / (2 * h)
            assert abs(fd - gr[e, c]) < 1e-6 * max(1.0, abs(fd))
    k = (2, 4, 1)
    d = np.zeros_like(V)
    d[k] = h
    assert abs((S(V_=V + d) - S(V_=V - d)) / (2 * h) - gV[k]) < 1e-6
    k = (3, 7, 0)
    d = np.zeros_like(w)
    d[k] = h
    assert abs((S(w_=w + d) - S(w_=w - d)) / (2 * h) - gw[k]) < 1e-6
