"""Pins of the oracle's spherical harmonics and Clebsch-Gordan table.

Every check compares the oracle with something other than itself: closed
forms, textbook tables (tests/golden), scipy / sympy library routines,
invariants (addition theorem, orthonormality, completeness, product rule),
rotation equivariance and a brute-force null-space solve.
"""
import math
import os

import numpy as np
import pytest
from scipy.spatial.transform import Rotation
from scipy.special import eval_legendre, sph_harm_y
from sympy.physics.wigner import clebsch_gordan

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def unit_points(n, seed):
    g = np.random.default_rng(seed)
    v = g.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def sh_block(L, pts, l):
    Y = oracle.sh(L, pts)
    return Y[:, l * l:(l + 1) ** 2]


def wigner_D(l, R, npts=80, seed=3):
    """D^l(R) from Y_l(R n) = D Y_l(n), least squares over npts directions."""
    n = unit_points(npts, seed)
    A = sh_block(l, n, l)
    B = sh_block(l, n @ R.T, l)
    Dt, *_ = np.linalg.lstsq(A, B, rcond=None)
    return Dt.T


# ---------------------------------------------------------------- SH ------

@pytest.mark.parametrize("L", [0, 1, 2, 3, 4])
def test_sh_pole(L):
    Y = oracle.sh(L, np.array([[0.0, 0.0, 2.5]]))[0]
    for l in range(L + 1):
        for m in range(-l, l + 1):
            expect = math.sqrt(2 * l + 1) if m == 0 else 0.0
            assert abs(Y[l * l + l + m] - expect) < 1e-14


def test_sh_l1_l2_closed_forms():
    pts = unit_points(50, 1) * 1.7
    Y = oracle.sh(2, pts)
    n = pts / np.linalg.norm(pts, axis=1, keepdims=True)
    x, y, z = n.T
    s3, s5, s15 = math.sqrt(3), math.sqrt(5), math.sqrt(15)
    np.testing.assert_allclose(Y[:, 0], 1.0, atol=1e-14)
    np.testing.assert_allclose(Y[:, 1:4], s3 * np.stack([y, z, x], 1), atol=1e-13)
    ref2 = np.stack([s15 * x * y, s15 * y * z, s5 / 2 * (3 * z * z - 1), s15 * x * z,
                     s15 / 2 * (x * x - y * y)], 1)
    np.testing.assert_allclose(Y[:, 4:9], ref2, atol=1e-13)


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_sh_vs_scipy_complex(L):
    """Real component-normalised SH from scipy's orthonormal complex SH (CS phase):
    m>0: sqrt2 (-1)^m Re Y_l^m, m<0: sqrt2 (-1)^m Im Y_l^|m|, times sqrt(4 pi)."""
    pts = unit_points(40, 2)
    Y = oracle.sh(L, pts)
    theta = np.arccos(np.clip(pts[:, 2], -1, 1))
    phi = np.arctan2(pts[:, 1], pts[:, 0])
    for l in range(L + 1):
        for m in range(-l, l + 1):
            c = sph_harm_y(l, abs(m), theta, phi) * math.sqrt(4 * math.pi)
            if m > 0:
                ref = math.sqrt(2) * (-1) ** m * c.real
            elif m == 0:
                ref = c.real
            else:
                ref = math.sqrt(2) * (-1) ** m * c.imag
            np.testing.assert_allclose(Y[:, l * l + l + m], ref, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_sh_norm_and_addition_theorem(L):
    a = unit_points(30, 4)
    b = unit_points(30, 5)
    Ya, Yb = oracle.sh(L, a), oracle.sh(L, b)
    for l in range(L + 1):
        sl = slice(l * l, (l + 1) ** 2)
        np.testing.assert_allclose((Ya[:, sl] ** 2).sum(1), 2 * l + 1, rtol=1e-13)
        lhs = (Ya[:, sl] * Yb[:, sl]).sum(1)
        rhs = (2 * l + 1) * eval_legendre(l, (a * b).sum(1))
        np.testing.assert_allclose(lhs, rhs, atol=1e-12)


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_sh_gradient_fd_and_homogeneity(L):
    g = np.random.default_rng(7)
    for _ in range(6):
        r = g.standard_normal(3) * g.uniform(0.8, 6.0)
        v = g.standard_normal(3)
        Y, dY, HV = oracle.sh_point(L, r, v)
        h = 1e-6 * np.linalg.norm(r)
        for k in range(3):
            e = np.zeros(3)
            e[k] = h
            fd = (oracle.sh_point(L, r + e)[0] - oracle.sh_point(L, r - e)[0]) / (2 * h)
            np.testing.assert_allclose(dY[k], fd, atol=2e-8 * (1 + np.abs(fd).max()))
            # HV_k = d/dr_k (grad Y . v)
            gp = oracle.sh_point(L, r + e)[1].T @ v
            gm = oracle.sh_point(L, r - e)[1].T @ v
            np.testing.assert_allclose(HV[k], (gp - gm) / (2 * h), atol=2e-7 * (1 + np.abs(HV).max()))
        # degree-0 homogeneity: Y(s r) = Y(r) and r . grad Y = 0
        np.testing.assert_allclose(oracle.sh_point(L, 3.3 * r)[0], Y, atol=1e-13)
        np.testing.assert_allclose(r @ dY, 0.0, atol=1e-12)


def test_wigner_D_l1_closed_form_and_homomorphism():
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], float)   # (x,y,z) -> (y,z,x)
    R1 = Rotation.random(random_state=11).as_matrix()
    R2 = Rotation.random(random_state=12).as_matrix()
    np.testing.assert_allclose(wigner_D(1, R1), P @ R1 @ P.T, atol=1e-12)
    for l in range(5):
        D1, D2, D12 = wigner_D(l, R1), wigner_D(l, R2), wigner_D(l, R1 @ R2)
        np.testing.assert_allclose(D1 @ D1.T, np.eye(2 * l + 1), atol=1e-11)
        np.testing.assert_allclose(D12, D1 @ D2, atol=1e-11)


# ---------------------------------------------------------------- CG ------

def _golden_j2_1():
    rows = []
    with open(os.path.join(GOLDEN, "cg_j2_1.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            dJ, m2, expr = [t.strip() for t in line.split("|")]
            rows.append((int(dJ), int(m2), expr))
    return rows


def test_cg_complex_textbook_table():
    rows = _golden_j2_1()
    assert len(rows) == 9
    n = 0
    for j1 in range(1, 8):
        for dJ, m2, expr in rows:
            J = j1 + dJ
            for M in range(-J, J + 1):
                m1 = M - m2
                if abs(m1) > j1:
                    continue
                ref = eval(expr, {"__builtins__": {}}, {"sqrt": math.sqrt, "j1": j1, "M": M})
                got = oracle.cg_complex(j1, m1, 1, m2, J, M)
                assert abs(got - ref) < 1e-13, (j1, m1, m2, J, M, got, ref)
                n += 1
    assert n > 200


def test_cg_complex_vs_sympy():
    for j1 in range(5):
        for j2 in range(5):
            for J in range(abs(j1 - j2), j1 + j2 + 1):
                for m1 in range(-j1, j1 + 1):
                    for m2 in range(-j2, j2 + 1):
                        M = m1 + m2
                        if abs(M) > J:
                            continue
                        ref = float(clebsch_gordan(j1, j2, J, m1, m2, M))
                        assert abs(oracle.cg_complex(j1, m1, j2, m2, J, M) - ref) < 1e-13


def all_paths(L):
    return [tuple(p) for p in oracle.paths(L)]


def test_path_counts_and_order():
    expect = {1: 5, 2: 15, 3: 34, 4: 65}
    for L, P in expect.items():
        ps = all_paths(L)
        assert len(ps) == P
        assert ps == sorted(ps)
        for l1, l2, l3 in ps:
            assert abs(l1 - l2) <= l3 <= min(l1 + l2, L)
    assert [oracle.dims(L)["nnz"] for L in range(1, 5)] == [16, 137, 611, 2052]
    assert [oracle.dims(L)["Dout"] for L in range(1, 5)] == [11, 51, 156, 375]


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_cg_real_part_rule_and_orthonormality(L):
    for l1, l2, l3 in all_paths(L):
        C, disc = oracle.cg_real_dense(l1, l2, l3)
        assert disc < 1e-15
        M = C.reshape(-1, 2 * l3 + 1)
        np.testing.assert_allclose(M.T @ M, np.eye(2 * l3 + 1), atol=1e-13)


@pytest.mark.parametrize("l1,l2", [(0, 3), (1, 1), (1, 2), (2, 2), (1, 4), (3, 3), (4, 4)])
def test_cg_completeness(l1, l2):
    d = (2 * l1 + 1) * (2 * l2 + 1)
    S = np.zeros((d, d))
    for l3 in range(abs(l1 - l2), l1 + l2 + 1):
        C, _ = oracle.cg_real_dense(l1, l2, l3)
        M = C.reshape(d, -1)
        S += M @ M.T
    np.testing.assert_allclose(S, np.eye(d), atol=1e-13)


def test_cg_special_cases():
    s = 1 / math.sqrt(2)
    for l in range(5):
        C, _ = oracle.cg_real_dense(0, l, l)
        np.testing.assert_allclose(C[0], np.eye(2 * l + 1), atol=1e-14)
        C, _ = oracle.cg_real_dense(l, 0, l)
        np.testing.assert_allclose(C[:, 0, :], np.eye(2 * l + 1), atol=1e-14)
        C, _ = oracle.cg_real_dense(l, l, 0)
        np.testing.assert_allclose(C[:, :, 0], (-1) ** l * np.eye(2 * l + 1) / math.sqrt(2 * l + 1),
                                   atol=1e-14)
    # 1 x 1 -> 1 is the cross product / sqrt2 in (y, z, x) component order
    C, _ = oracle.cg_real_dense(1, 1, 1)
    g = np.random.default_rng(0)
    a, b = g.standard_normal(3), g.standard_normal(3)
    yzx = [1, 2, 0]
    got = np.einsum("abc,a,b->c", C, a[yzx], b[yzx])
    np.testing.assert_allclose(got, np.cross(a, b)[yzx] * s, atol=1e-14)


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_cg_product_rule(L):
    """sum C Y_l1(n) Y_l2(n) = sqrt((2l1+1)(2l2+1)/(2l3+1)) <l1 0 l2 0|l3 0> Y_l3(n)
    (zero for odd l1+l2+l3), with <..|..> from sympy."""
    pts = unit_points(20, 9)
    Y = oracle.sh(L, pts)
    for l1, l2, l3 in all_paths(L):
        C, _ = oracle.cg_real_dense(l1, l2, l3)
        Y1 = Y[:, l1 * l1:(l1 + 1) ** 2]
        Y2 = Y[:, l2 * l2:(l2 + 1) ** 2]
        Y3 = Y[:, l3 * l3:(l3 + 1) ** 2]
        lhs = np.einsum("abc,na,nb->nc", C, Y1, Y2)
        k = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * l3 + 1)) * float(
            clebsch_gordan(l1, l2, l3, 0, 0, 0))
        np.testing.assert_allclose(lhs, k * Y3, atol=1e-12)


@pytest.mark.parametrize("L", [2, 4])
def test_cg_equivariance(L):
    Rs = [Rotation.random(random_state=s).as_matrix() for s in (21, 22)]
    for R in Rs:
        D = [wigner_D(l, R) for l in range(L + 1)]
        for l1, l2, l3 in all_paths(L):
            C, _ = oracle.cg_real_dense(l1, l2, l3)
            lhs = np.einsum("abc,ax,by->xyc", C, D[l1], D[l2])   # C(D1 (x) D2)
            rhs = np.einsum("xyc,dc->xyd", C, D[l3])             # D3 C
            np.testing.assert_allclose(lhs, rhs, atol=1e-11)


def test_cg_nullspace_brute_force():
    """The equivariant maps l1 (x) l2 -> l3 form a 1-D space; the oracle's
    tensor is (up to sign) its unit vector."""
    L = 3
    Rs = [Rotation.random(random_state=s).as_matrix() for s in (31, 32, 33)]
    Ds = [[wigner_D(l, R) for l in range(L + 1)] for R in Rs]
    for l1, l2, l3 in all_paths(L):
        d1, d2, d3 = 2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1
        n = d1 * d2 * d3
        cols = []
        for k in range(n):                                   # the constraint map on a basis
            T = np.zeros(n)
            T[k] = 1.0
            T = T.reshape(d1, d2, d3)
            r = [np.einsum("abc,ax,by->xyc", T, D[l1], D[l2]) - np.einsum("xyc,dc->xyd", T, D[l3])
                 for D in Ds]
            cols.append(np.concatenate([q.reshape(-1) for q in r]))
        A = np.stack(cols, 1)
        _, s, vt = np.linalg.svd(A)
        rank = int((s > 1e-9).sum())
        assert n - rank == 1, (l1, l2, l3, s[-3:])
        null = vt[-1]
        C, _ = oracle.cg_real_dense(l1, l2, l3)
        c = C.reshape(-1)
        c = c / np.linalg.norm(c)
        assert abs(abs(c @ null) - 1) < 1e-10


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_sparse_table_matches_dense(L):
    ptr, m, val = oracle.cg_sparse(L)
    ps = all_paths(L)
    assert ptr.shape[0] == len(ps) + 1
    for p, (l1, l2, l3) in enumerate(ps):
        C, _ = oracle.cg_real_dense(l1, l2, l3)
        idx = np.argwhere(np.abs(C) > 1e-12)            # row-major = (m1, m2, m3) order
        got = m[ptr[p]:ptr[p + 1]].astype(int) + np.array([l1, l2, l3])
        np.testing.assert_array_equal(got, idx)
        np.testing.assert_array_equal(val[ptr[p]:ptr[p + 1]], C[tuple(idx.T)])
    assert np.abs(val).min() > 0.07
