"""Pins for the oracle's node-local correlation product (the weighted product
ladder B_{k+1} = sum_p W_k[p] CG_p(B_k, A), out = B_1 + ... + B_nu):

  * nu = 1 is the identity;
  * l_max = 0 and inputs with only l = 0 are scalar polynomials in closed form;
  * a pure vector input at nu = 2: the l = 0 block is -W |a|^2 / sqrt3, the
    l = 1 block keeps only a (a x a = 0), and the l = 2 block carries the rest
    of |a|^4 (the coupling is orthogonal);
  * the whole ladder against a dense recursion whose CG comes from sympy;
  * rotation equivariance;
  * the VJP with respect to A: central differences of <G, out>, the
    derivative of the l_max = 0 polynomial, and rotation covariance.
"""
import math

import numpy as np
import pytest
from scipy.spatial.transform import Rotation

import oracle
from test_oracle_conv import _library_dense_cg, _wigner_D


def paths(L):
    return [tuple(int(v) for v in p) for p in oracle.paths(L)]


def test_order_one_is_identity():
    A = np.random.default_rng(0).standard_normal((4, 16, 3))
    assert np.array_equal(oracle.node_product(3, A, None, 1), A)


@pytest.mark.parametrize("nu", [2, 3, 5])
def test_scalar_closed_form(nu):
    """l_max = 0: B_{k+1} = W_k B_k a, so out = sum_k (prod_{j<k} W_j) a^k."""
    g = np.random.default_rng(nu)
    A = g.standard_normal((6, 1, 4))
    W = g.standard_normal((nu - 1, 1, 4))
    out = oracle.node_product(0, A, W, nu)
    a = A[:, 0, :]
    want, term = a.copy(), a.copy()
    for k in range(nu - 1):
        term = W[k, 0] * term * a
        want += term
    np.testing.assert_allclose(out[:, 0, :], want, rtol=1e-13, atol=1e-13)


def test_scalar_input_stays_scalar():
    """Only l = 0 populated at l_max = 2: the ladder only uses the (0, 0, 0) path."""
    g = np.random.default_rng(1)
    A = np.zeros((5, 9, 3))
    A[:, 0, :] = g.standard_normal((5, 3))
    W = g.standard_normal((3, 15, 3))
    out = oracle.node_product(2, A, W, 4)
    p000 = paths(2).index((0, 0, 0))
    a = A[:, 0, :]
    want, term = a.copy(), a.copy()
    for k in range(3):
        term = W[k, p000] * term * a
        want += term
    np.testing.assert_allclose(out[:, 0, :], want, rtol=1e-13, atol=1e-13)
    assert np.abs(out[:, 1:, :]).max() == 0.0


def test_pure_vector_order_two():
    g = np.random.default_rng(2)
    n, C = 6, 3
    A = np.zeros((n, 9, C))
    A[:, 1:4, :] = g.standard_normal((n, 3, C))
    W = g.standard_normal((1, 15, C))
    out = oracle.node_product(2, A, W, 2)
    P = paths(2)
    a2 = (A[:, 1:4, :] ** 2).sum(axis=1)                       # |a|^2 per (node, channel)
    np.testing.assert_allclose(out[:, 0, :], -W[0, P.index((1, 1, 0))] * a2 / math.sqrt(3), atol=1e-13)
    np.testing.assert_allclose(out[:, 1:4, :], A[:, 1:4, :], atol=1e-13)   # a x a = 0
    l2 = out[:, 4:9, :] / W[0, P.index((1, 1, 2))]
    np.testing.assert_allclose((l2 ** 2).sum(axis=1), 2.0 / 3.0 * a2 ** 2, rtol=1e-12)


@pytest.mark.parametrize("L,nu", [(1, 4), (2, 3)])
def test_ladder_against_sympy_recursion(L, nu):
    g = np.random.default_rng(10 + L)
    n, C = 3, 2
    D = (L + 1) ** 2
    A = g.standard_normal((n, D, C))
    W = g.standard_normal((nu - 1, len(paths(L)), C))
    out = oracle.node_product(L, A, W, nu)
    T = {p: _library_dense_cg(*p) for p in paths(L)}
    B, want = A.copy(), A.copy()
    for k in range(nu - 1):
        nb = np.zeros_like(A)
        for q, (l1, l2, l3) in enumerate(paths(L)):
            nb[:, l3 * l3:(l3 + 1) ** 2] += W[k, q] * np.einsum(
                "abc,nau,nbu->ncu", T[(l1, l2, l3)], B[:, l1 * l1:(l1 + 1) ** 2], A[:, l2 * l2:(l2 + 1) ** 2])
        B = nb
        want += B
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("L", [2, 3])
def test_rotation_equivariance(L):
    g = np.random.default_rng(20 + L)
    n, C, nu = 4, 3, 4
    D = (L + 1) ** 2
    A = g.standard_normal((n, D, C)) * 0.5
    W = g.standard_normal((nu - 1, len(paths(L)), C))
    R = Rotation.random(random_state=30 + L).as_matrix()

    def rot(x):
        y = np.empty_like(x)
        for l in range(L + 1):
            y[:, l * l:(l + 1) ** 2] = np.einsum("ab,nbu->nau", _wigner_D(l, R), x[:, l * l:(l + 1) ** 2])
        return y

    lhs = oracle.node_product(L, rot(A), W, nu)
    rhs = rot(oracle.node_product(L, A, W, nu))
    np.testing.assert_allclose(lhs, rhs, atol=1e-9 * np.abs(rhs).max())


@pytest.mark.parametrize("L,nu", [(1, 3), (2, 4), (3, 2)])
def test_vjp_finite_differences(L, nu):
    g = np.random.default_rng(40 + L)
    n, C = 3, 2
    D = (L + 1) ** 2
    A = g.standard_normal((n, D, C)) * 0.7
    W = g.standard_normal((nu - 1, len(paths(L)), C))
    G = g.standard_normal((n, D, C))
    gA = oracle.node_product_vjp(L, A, W, G, nu)
    h = 1e-6
    for idx in [(0, 0, 0), (1, D - 1, 1), (2, D // 2, 0), (0, 1, 1)]:
        d = np.zeros_like(A)
        d[idx] = h
        fd = ((G * oracle.node_product(L, A + d, W, nu)).sum() - (G * oracle.node_product(L, A - d, W, nu)).sum()) / (2 * h)
        assert abs(fd - gA[idx]) < 1e-6 * max(1.0, abs(fd)), (idx, fd, gA[idx])


def test_vjp_scalar_polynomial():
    """l_max = 0: out = sum_k c_k a^k with c_k = prod_{j<k-1} W_j, so gA = G sum_k k c_k a^(k-1)."""
    g = np.random.default_rng(50)
    nu = 4
    A = g.standard_normal((5, 1, 3))
    W = g.standard_normal((nu - 1, 1, 3))
    G = g.standard_normal((5, 1, 3))
    gA = oracle.node_product_vjp(0, A, W, G, nu)
    a = A[:, 0, :]
    c, want = np.ones_like(a), np.zeros_like(a)
    for k in range(1, nu + 1):
        want += k * c * a ** (k - 1)
        if k < nu:
            c = c * W[k - 1, 0]
    np.testing.assert_allclose(gA[:, 0, :], G[:, 0, :] * want, rtol=1e-12, atol=1e-12)


def test_vjp_rotation_covariance():
    L, nu = 2, 3
    g = np.random.default_rng(60)
    n, C = 3, 2
    A = g.standard_normal((n, 9, C)) * 0.6
    W = g.standard_normal((nu - 1, 15, C))
    G = g.standard_normal((n, 9, C))
    R = Rotation.random(random_state=61).as_matrix()

    def rot(x):
        y = np.empty_like(x)
        for l in range(L + 1):
            y[:, l * l:(l + 1) ** 2] = np.einsum("ab,nbu->nau", _wigner_D(l, R), x[:, l * l:(l + 1) ** 2])
        return y

    lhs = oracle.node_product_vjp(L, rot(A), W, rot(G), nu)
    np.testing.assert_allclose(lhs, rot(oracle.node_product_vjp(L, A, W, G, nu)), atol=1e-9)


# ------------------------------------------------------- weight gradient

def _case(L, nu, n=3, C=2, seed=0):
    g = np.random.default_rng(seed)
    P = len(paths(L))
    A = g.standard_normal((n, (L + 1) ** 2, C))
    W = g.standard_normal((nu - 1, P, C)) / math.sqrt(P)
    G = g.standard_normal((n, (L + 1) ** 2, C))
    return A, W, G


@pytest.mark.parametrize("L,nu", [(1, 2), (2, 3), (3, 4), (2, 5)])
def test_wgrad_euler_identity(L, nu):
    """B_k is homogeneous of degree k - 1 in the weights, so
    <gW, W> = sum_{k >= 2} (k - 1) <G, B_k>, with B_k = out(nu = k) - out(nu = k - 1)
    from the forward ladder."""
    A, W, G = _case(L, nu, seed=L + nu)
    gW = oracle.node_product_wgrad(L, A, W, G, nu)
    lhs = (gW * W).sum()
    rhs = 0.0
    prev = oracle.node_product(L, A, None, 1)
    for k in range(2, nu + 1):
        cur = oracle.node_product(L, A, W[:k - 1], k)
        rhs += (k - 1) * (G * (cur - prev)).sum()
        prev = cur
    assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(rhs))


@pytest.mark.parametrize("L,nu", [(2, 3), (3, 4)])
def test_wgrad_finite_differences(L, nu):
    """Central differences of <G, out> in single weights (every step, several paths)."""
    A, W, G = _case(L, nu, seed=7 * L + nu)
    gW = oracle.node_product_wgrad(L, A, W, G, nu)
    g = np.random.default_rng(11)
    h = 1e-5
    for _ in range(12):
        idx = tuple(int(g.integers(0, s)) for s in W.shape)
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += h
        Wm[idx] -= h
        fd = ((G * oracle.node_product(L, A, Wp, nu)).sum() - (G * oracle.node_product(L, A, Wm, nu)).sum()) / (2 * h)
        assert abs(fd - gW[idx]) < 1e-7 * max(1.0, abs(fd)), (idx, fd, gW[idx])


def test_wgrad_order_one_is_empty_and_additive():
    """nu = 1 has no weights; gW of a batch is the sum of the per-node gW."""
    A, W, G = _case(2, 1)
    assert oracle.node_product_wgrad(2, A, None, G, 1).size == 0
    A, W, G = _case(2, 3, n=4, seed=5)
    whole = oracle.node_product_wgrad(2, A, W, G, 3)
    parts = sum(oracle.node_product_wgrad(2, A[i:i + 1], W, G[i:i + 1], 3) for i in range(4))
    np.testing.assert_allclose(whole, parts, rtol=1e-12, atol=1e-12)
