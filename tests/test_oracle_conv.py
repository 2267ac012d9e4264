"""Pins of the oracle's convolution (forward, VJP, VJP-of-VJP) and transpose.

Checks: single-path closed forms, a dense brute force built from library
routines (sympy complex CG, scipy complex SH, a textbook change of basis),
rotation equivariance, permutation invariance, linearity / adjoint
identities, finite differences in float64, and a brute-force stable sort.
"""
import math

import numpy as np
import pytest
from scipy.spatial.transform import Rotation
from scipy.special import sph_harm_y
from sympy.physics.wigner import clebsch_gordan

import oracle
import workloads

YZX = [1, 2, 0]


def wl(L, C, n=7, k=5, seed=0, empty_rows=True):
    return workloads.small(L, C, n, k, seed=seed, empty_rows=empty_rows)


def arrays(w, dtype=np.float64):
    return (w.row_ptr, w.src, w.vec.astype(dtype), w.x.astype(dtype), w.w.astype(dtype))


def path_index(L):
    return {tuple(p): i for i, p in enumerate(oracle.paths(L))}


def out_block(L, p):
    ps = oracle.paths(L)
    off = sum(2 * int(q[2]) + 1 for q in ps[:p])
    return slice(off, off + 2 * int(ps[p][2]) + 1)


def edge_dst(row_ptr):
    return np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))


# --------------------------------------------------------- closed forms ----

def test_fwd_single_path_closed_forms():
    L, C = 2, 3
    w = wl(L, C, n=9, k=6, seed=1)
    rp, src, vec, x, W = arrays(w)
    pidx = path_index(L)
    dst = edge_dst(rp)
    n = vec / np.linalg.norm(vec, axis=1, keepdims=True)
    Y = oracle.sh(L, vec)

    def only(p):
        Wp = np.zeros_like(W)
        Wp[:, p] = W[:, p]
        return oracle.fwd(L, rp, src, vec, x, Wp)

    # (0, l, l): out = sum_e w x0 Y_l(n_e)
    for l in range(L + 1):
        p = pidx[(0, l, l)]
        out = only(p)[:, out_block(L, p)]
        ref = np.zeros_like(out)
        for e in range(len(src)):
            ref[dst[e]] += W[e, p][None, :] * x[src[e], 0][None, :] * Y[e, l * l:(l + 1) ** 2][:, None]
        np.testing.assert_allclose(out, ref, atol=1e-12)
    # (1, 1, 0): out = -sum_e w (xvec . n)
    p = pidx[(1, 1, 0)]
    out = only(p)[:, out_block(L, p)]
    ref = np.zeros_like(out)
    for e in range(len(src)):
        xv = x[src[e], 1:4][np.argsort(YZX)]       # rows (y, z, x) -> (x, y, z)
        ref[dst[e], 0] += -W[e, p] * (xv * n[e][:, None]).sum(0)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    # (1, 1, 1): out = sqrt(3/2) sum_e w (xvec x n), (y, z, x) order
    p = pidx[(1, 1, 1)]
    out = only(p)[:, out_block(L, p)]
    ref = np.zeros_like(out)
    for e in range(len(src)):
        xv = x[src[e], 1:4][np.argsort(YZX)]
        cr = np.cross(xv.T, n[e][None, :]).T         # (3, C) in xyz
        ref[dst[e]] += math.sqrt(1.5) * W[e, p][None, :] * cr[YZX]
    np.testing.assert_allclose(out, ref, atol=1e-12)


def _U(l):
    """Textbook complex -> real change of basis, row m' (real), column m (complex)."""
    d = 2 * l + 1
    U = np.zeros((d, d), complex)
    h = 1 / math.sqrt(2)
    for mp in range(-l, l + 1):
        if mp > 0:
            U[mp + l, -mp + l] = h
            U[mp + l, mp + l] = (-1) ** mp * h
        elif mp == 0:
            U[l, l] = 1
        else:
            k = -mp
            U[mp + l, mp + l] = 1j * h
            U[mp + l, k + l] = -1j * (-1) ** k * h
    return U


def _library_dense_cg(l1, l2, l3):
    Cc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            if abs(m1 + m2) <= l3:
                Cc[m1 + l1, m2 + l2, m1 + m2 + l3] = float(clebsch_gordan(l1, l2, l3, m1, m2, m1 + m2))
    T = np.einsum("cg,abg,xa,yb->xyc", _U(l3), Cc, _U(l1).conj(), _U(l2).conj())
    return T.imag if (l1 + l2 + l3) % 2 else T.real


def _library_sh(L, vec):
    n = vec / np.linalg.norm(vec, axis=1, keepdims=True)
    th = np.arccos(np.clip(n[:, 2], -1, 1))
    ph = np.arctan2(n[:, 1], n[:, 0])
    Y = np.zeros((len(vec), (L + 1) ** 2))
    for l in range(L + 1):
        for m in range(-l, l + 1):
            c = sph_harm_y(l, abs(m), th, ph) * math.sqrt(4 * math.pi)
            Y[:, l * l + l + m] = (c.real if m == 0 else
                                   math.sqrt(2) * (-1) ** m * (c.real if m > 0 else c.imag))
    return Y


@pytest.mark.parametrize("L", [1, 2, 3])
def test_fwd_dense_library_brute_force(L):
    """Forward vs a dense einsum whose CG comes from sympy and whose SH come from scipy."""
    C = 2
    w = wl(L, C, n=6, k=4, seed=2)
    rp, src, vec, x, W = arrays(w)
    out = oracle.fwd(L, rp, src, vec, x, W)
    Y = _library_sh(L, vec)
    dst = edge_dst(rp)
    ref = np.zeros_like(out)
    for p, (l1, l2, l3) in enumerate(oracle.paths(L)):
        T = _library_dense_cg(int(l1), int(l2), int(l3))
        msg = np.einsum("abc,eb,eau,eu->ecu", T, Y[:, l2 * l2:(l2 + 1) ** 2],
                        x[src][:, l1 * l1:(l1 + 1) ** 2], W[:, p])
        np.add.at(ref[:, out_block(L, p)], dst, msg)
    np.testing.assert_allclose(out, ref, atol=1e-12)


# --------------------------------------------------------- symmetries ------

def _wigner_D(l, R):
    g = np.random.default_rng(3)
    n = g.standard_normal((80, 3))
    n /= np.linalg.norm(n, axis=1, keepdims=True)
    A = oracle.sh(l, n)[:, l * l:]
    B = oracle.sh(l, n @ R.T)[:, l * l:]
    return np.linalg.lstsq(A, B, rcond=None)[0].T


def _rot_x(L, R, x):
    y = np.empty_like(x)
    for l in range(L + 1):
        y[:, l * l:(l + 1) ** 2] = np.einsum("ab,nbu->nau", _wigner_D(l, R), x[:, l * l:(l + 1) ** 2])
    return y


def _rot_out(L, R, out):
    y = np.empty_like(out)
    for p, (l1, l2, l3) in enumerate(oracle.paths(L)):
        b = out_block(L, p)
        y[:, b] = np.einsum("ab,nbu->nau", _wigner_D(int(l3), R), out[:, b])
    return y


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_fwd_rotation_equivariance(L):
    w = wl(L, 3, n=6, k=4, seed=4)
    rp, src, vec, x, W = arrays(w)
    R = Rotation.random(random_state=40 + L).as_matrix()
    out = oracle.fwd(L, rp, src, vec, x, W)
    out_r = oracle.fwd(L, rp, src, vec @ R.T, _rot_x(L, R, x), W)
    np.testing.assert_allclose(out_r, _rot_out(L, R, out), atol=1e-10)


def test_fwd_permutation_invariance_and_relabel():
    L = 2
    w = wl(L, 3, n=8, k=6, seed=5)
    rp, src, vec, x, W = arrays(w)
    out = oracle.fwd(L, rp, src, vec, x, W)
    g = np.random.default_rng(1)
    # shuffle neighbour order inside each row (edge arrays permute along)
    perm = np.concatenate([rp[i] + g.permutation(rp[i + 1] - rp[i]) for i in range(len(rp) - 1)])
    out2 = oracle.fwd(L, rp, src[perm], vec[perm], x, W[perm])
    np.testing.assert_allclose(out2, out, atol=1e-12)
    # relabel nodes: sigma maps old id -> new id
    n = len(rp) - 1
    sigma = g.permutation(n)
    inv = np.argsort(sigma)
    rows = [np.arange(rp[inv[i]], rp[inv[i] + 1]) for i in range(n)]
    eorder = np.concatenate(rows).astype(np.int64)
    rp2 = np.zeros(n + 1, np.int32)
    rp2[1:] = np.cumsum([len(r) for r in rows])
    x2 = np.empty_like(x)
    x2[sigma] = x
    out3 = oracle.fwd(L, rp2, sigma[src[eorder]].astype(np.int32), vec[eorder], x2, W[eorder])
    np.testing.assert_allclose(out3[sigma], out, atol=1e-12)


# --------------------------------------------------------------- VJP -------

@pytest.mark.parametrize("L", [1, 2, 3])
def test_vjp_adjoint_identities(L):
    w = wl(L, 3, n=7, k=5, seed=6)
    rp, src, vec, x, W = arrays(w)
    G = w.G.astype(np.float64)
    gx, gw, gr = oracle.vjp(L, rp, src, vec, x, W, G)
    out = oracle.fwd(L, rp, src, vec, x, W)
    # forward is linear in x and in w: <G, F(x, w)> = <gx, x> = <gw, w>
    s = (G * out).sum()
    assert abs((gx * x).sum() - s) < 1e-10 * (1 + abs(s))
    assert abs((gw * W).sum() - s) < 1e-10 * (1 + abs(s))
    dx = np.random.default_rng(2).standard_normal(x.shape)
    assert abs((G * oracle.fwd(L, rp, src, vec, dx, W)).sum() - (gx * dx).sum()) < 1e-10 * (1 + abs(s))


@pytest.mark.parametrize("L", [1, 2, 3, 4])
def test_vjp_force_fd(L):
    w = wl(L, 2, n=5, k=3, seed=7)
    rp, src, vec, x, W = arrays(w)
    G = w.G.astype(np.float64)
    gx, gw, gr = oracle.vjp(L, rp, src, vec, x, W, G)
    E = len(src)
    for e in range(E):
        for k in range(3):
            h = 1e-6 * np.linalg.norm(vec[e])
            vp, vm = vec.copy(), vec.copy()
            vp[e, k] += h
            vm[e, k] -= h
            fd = ((G * oracle.fwd(L, rp, src, vp, x, W)).sum()
                  - (G * oracle.fwd(L, rp, src, vm, x, W)).sum()) / (2 * h)
            assert abs(fd - gr[e, k]) < 1e-6 * (1 + abs(fd)), (e, k, fd, gr[e, k])


def test_vjp_force_rotation_covariance():
    L = 2
    w = wl(L, 3, n=6, k=4, seed=8)
    rp, src, vec, x, W = arrays(w)
    G = w.G.astype(np.float64)
    R = Rotation.random(random_state=80).as_matrix()
    gx, gw, gr = oracle.vjp(L, rp, src, vec, x, W, G)
    gx2, gw2, gr2 = oracle.vjp(L, rp, src, vec @ R.T, _rot_x(L, R, x), W, _rot_out(L, R, G))
    np.testing.assert_allclose(gr2, gr @ R.T, atol=1e-10)
    np.testing.assert_allclose(gw2, gw, atol=1e-10)
    np.testing.assert_allclose(gx2, _rot_x(L, R, gx), atol=1e-10)


# -------------------------------------------------------------- VJP2 -------

def _vjp_scalar(L, rp, src, vec, x, W, G, Xp, Wp, Rp):
    gx, gw, gr = oracle.vjp(L, rp, src, vec, x, W, G)
    return (Xp * gx).sum() + (Wp * gw).sum() + (Rp * gr).sum()


@pytest.mark.parametrize("L", [2, 3])
def test_vjp2_finite_differences(L):
    """VJP2 outputs are the gradient of S = <X',gx> + <W',gw> + <R',gr>."""
    w = wl(L, 2, n=4, k=3, seed=9, empty_rows=False)
    rp, src, vec, x, W = arrays(w)
    G = w.G.astype(np.float64)
    Xp, Wp, Rp = w.ggx.astype(np.float64), w.ggw.astype(np.float64), w.ggvec.astype(np.float64)
    dx, dw, dr, dG = oracle.vjp2(L, rp, src, vec, x, W, G, Xp, Wp, Rp)
    g = np.random.default_rng(10)

    def S(**kw):
        a = dict(vec=vec, x=x, W=W, G=G)
        a.update(kw)
        return _vjp_scalar(L, rp, src, a["vec"], a["x"], a["W"], a["G"], Xp, Wp, Rp)

    # directional derivatives along random directions (x, w, G enter S polynomially)
    for name, val, grad in (("x", x, dx), ("W", W, dw), ("G", G, dG)):
        d = g.standard_normal(val.shape)
        h = 1e-4
        fd = (S(**{name: val + h * d}) - S(**{name: val - h * d})) / (2 * h)
        an = (grad * d).sum()
        assert abs(fd - an) < 1e-7 * (1 + abs(an)), (name, fd, an)
    for e in range(len(src)):
        for k in range(3):
            h = 1e-5 * np.linalg.norm(vec[e])
            vp, vm = vec.copy(), vec.copy()
            vp[e, k] += h
            vm[e, k] -= h
            fd = (S(vec=vp) - S(vec=vm)) / (2 * h)
            assert abs(fd - dr[e, k]) < 2e-6 * (1 + abs(fd)), (e, k, fd, dr[e, k])


def test_vjp2_linearity_pins():
    L = 2
    w = wl(L, 3, n=7, k=5, seed=11)
    rp, src, vec, x, W = arrays(w)
    G = w.G.astype(np.float64)
    Xp, Wp = w.ggx.astype(np.float64), w.ggw.astype(np.float64)
    # X' alone: dG = F(x := X'), dw = gw(x := X'), dx = 0, dr uses only Z1
    dx, dw, dr, dG = oracle.vjp2(L, rp, src, vec, x, W, G, Xp=Xp)
    np.testing.assert_allclose(dG, oracle.fwd(L, rp, src, vec, Xp, W), atol=1e-11)
    np.testing.assert_allclose(dw, oracle.vjp(L, rp, src, vec, Xp, W, G)[1], atol=1e-11)
    np.testing.assert_allclose(dx, 0.0, atol=0)
    # W' alone: dG = F(w := W'), dx = gx(w := W'), dw = 0
    dx, dw, dr, dG = oracle.vjp2(L, rp, src, vec, x, W, G, Wp=Wp)
    np.testing.assert_allclose(dG, oracle.fwd(L, rp, src, vec, x, Wp), atol=1e-11)
    np.testing.assert_allclose(dx, oracle.vjp(L, rp, src, vec, x, Wp, G)[0], atol=1e-11)
    np.testing.assert_allclose(dw, 0.0, atol=0)
    # no cotangent at all: every output is zero
    outs = oracle.vjp2(L, rp, src, vec, x, W, G)
    for o in outs:
        np.testing.assert_allclose(o, 0.0, atol=0)


# --------------------------------------------------------- transpose -------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_transpose_vs_stable_sort(seed):
    w = wl(1, 1, n=40, k=12, seed=seed)
    rp, src = w.row_ptr, w.src
    sp, perm, pdst = oracle.transpose(rp, src, 40)
    order = np.argsort(src, kind="stable")
    np.testing.assert_array_equal(perm, order)
    np.testing.assert_array_equal(pdst, edge_dst(rp)[order])
    np.testing.assert_array_equal(sp, np.concatenate([[0], np.cumsum(np.bincount(src, minlength=40))]))


def test_transpose_empty_graph():
    sp, perm, pdst = oracle.transpose(np.zeros(4, np.int32), np.zeros(0, np.int32), 5)
    np.testing.assert_array_equal(sp, np.zeros(6, np.int32))
    assert perm.size == 0 and pdst.size == 0
