"""Pins for the oracle's edge-to-atom force assembly: the sign convention by
finite differences of a toy pair energy, zero net force, brute force."""
import numpy as np

import oracle
import workloads


def toy(vec):
    """A pair energy with a closed-form gradient: sum_e a . v_e + |v_e|^4 / 4."""
    a = np.array([0.3, -0.7, 0.2])
    E = (vec @ a).sum() + 0.25 * (np.einsum("ei,ei->e", vec, vec) ** 2).sum()
    grad = a[None, :] + np.einsum("ei,ei->e", vec, vec)[:, None] * vec
    return E, grad


def test_forces_are_minus_position_gradient():
    """vec_e = pos[src_e] - pos[dst_e]: central differences of the toy energy
    over every atom coordinate give -F."""
    g = np.random.default_rng(4)
    wl = workloads.small(1, 1, 9, 4, seed=2)
    pos = g.standard_normal((wl.n, 3))
    dst = np.repeat(np.arange(wl.n_dst), np.diff(wl.row_ptr))

    def energy(p):
        return toy(p[wl.src] - p[dst])[0]

    F = oracle.edge_forces(wl.row_ptr, wl.src, wl.n, toy(pos[wl.src] - pos[dst])[1])
    h = 1e-6
    for k in range(wl.n):
        for c in range(3):
            d = np.zeros_like(pos)
            d[k, c] = h
            fd = (energy(pos + d) - energy(pos - d)) / (2 * h)
            assert abs(F[k, c] + fd) < 1e-6 * max(1.0, abs(fd))


def test_net_force_vanishes():
    g = np.random.default_rng(5)
    wl = workloads.small(1, 1, 30, 8, seed=3)
    gr = g.standard_normal((wl.E, 3))
    F = oracle.edge_forces(wl.row_ptr, wl.src, wl.n, gr)
    assert np.abs(F.sum(axis=0)).max() < 1e-12 * np.abs(gr).sum()


def test_brute_force_per_atom():
    g = np.random.default_rng(6)
    wl = workloads.bipartite(1, 1, 6, 11, 0, 5, seed=1)      # n_dst != n_src
    gr = g.standard_normal((wl.E, 3))
    F = oracle.edge_forces(wl.row_ptr, wl.src, wl.n, gr)
    dst = np.repeat(np.arange(wl.n_dst), np.diff(wl.row_ptr))
    want = np.zeros((max(wl.n_dst, wl.n), 3))
    for e in range(wl.E):
        want[dst[e]] += gr[e]
        want[wl.src[e]] -= gr[e]
    assert np.abs(F - want).max() < 1e-13
