"""Pins for the oracle's channel mixing (the per-irrep linear layer after the
convolution): closed forms and an independently assembled dense product."""
import numpy as np
import pytest

import oracle


def offsets(L):
    p = oracle.paths(L)
    sizes = 2 * p[:, 2] + 1
    return p, np.concatenate([[0], np.cumsum(sizes)])


@pytest.mark.parametrize("L,C", [(0, 3), (1, 2), (2, 4), (3, 2), (4, 1)])
def test_identity_blocks_sum_paths(L, C):
    """W_l = n_l stacked identities: y sums the blocks of the paths of order l."""
    g = np.random.default_rng(L * 10 + C)
    p, off = offsets(L)
    out = g.standard_normal((3, off[-1], C))
    W = np.concatenate([np.tile(np.eye(C), (n, 1)).reshape(-1) for n in oracle.mix_rows(L)])
    y = oracle.channel_mix(L, out, W)
    want = np.zeros_like(y)
    for q, (l1, l2, l3) in enumerate(p):
        want[:, l3 * l3:(l3 + 1) * (l3 + 1), :] += out[:, off[q]:off[q + 1], :]
    assert np.abs(y - want).max() < 1e-12


@pytest.mark.parametrize("L,C", [(1, 3), (2, 2), (3, 2)])
def test_matches_assembled_matrix(L, C):
    """Against one dense product per order, with the input gathered into
    [(node, m), (path of order l, u)] rows in numpy."""
    g = np.random.default_rng(7 + L)
    p, off = offsets(L)
    n = 5
    out = g.standard_normal((n, off[-1], C))
    rows = oracle.mix_rows(L)
    Ws = [g.standard_normal((k * C, C)) for k in rows]
    y = oracle.channel_mix(L, out, np.concatenate([w.reshape(-1) for w in Ws]))
    for l, Wl in enumerate(Ws):
        qs = [q for q in range(len(p)) if p[q, 2] == l]
        A = np.concatenate([out[:, off[q]:off[q + 1], :] for q in qs], axis=2)  # [n, 2l+1, n_l*C]
        want = (A.reshape(-1, len(qs) * C) @ Wl).reshape(n, 2 * l + 1, C)
        assert np.abs(y[:, l * l:(l + 1) * (l + 1), :] - want).max() < 1e-12


def test_one_path_selected():
    """W_l zero except the block of one path: y is that block times the matrix."""
    L, C = 2, 3
    g = np.random.default_rng(3)
    p, off = offsets(L)
    out = g.standard_normal((2, off[-1], C))
    rows = oracle.mix_rows(L)
    target = 4                       # a path of order p[4, 2]
    l = int(p[target, 2])
    rank = int((p[:target, 2] == l).sum())
    M = g.standard_normal((C, C))
    Ws = [np.zeros((k * C, C)) for k in rows]
    Ws[l][rank * C:(rank + 1) * C] = M
    y = oracle.channel_mix(L, out, np.concatenate([w.reshape(-1) for w in Ws]))
    want = np.zeros_like(y)
    want[:, l * l:(l + 1) * (l + 1), :] = out[:, off[target]:off[target + 1], :] @ M
    assert np.abs(y - want).max() < 1e-12


def test_commutes_with_maps_on_components():
    """The same matrix for every component m: any per-order map A_l acting on
    the m index of all blocks of order l commutes with the mixing."""
    L, C = 3, 2
    g = np.random.default_rng(11)
    p, off = offsets(L)
    out = g.standard_normal((2, off[-1], C))
    W = g.standard_normal(sum(oracle.mix_rows(L)) * C * C)
    A = [g.standard_normal((2 * l + 1, 2 * l + 1)) for l in range(L + 1)]
    moved = out.copy()
    for q, (l1, l2, l3) in enumerate(p):
        moved[:, off[q]:off[q + 1], :] = np.einsum("ab,nbc->nac", A[l3], out[:, off[q]:off[q + 1], :])
    y = oracle.channel_mix(L, out, W)
    y_moved = oracle.channel_mix(L, moved, W)
    for l in range(L + 1):
        sl = slice(l * l, (l + 1) * (l + 1))
        assert np.abs(y_moved[:, sl] - np.einsum("ab,nbc->nac", A[l], y[:, sl])).max() < 1e-10


@pytest.mark.parametrize("L,C", [(1, 3), (2, 4), (3, 2), (4, 1)])
def test_vjp_is_the_adjoint(L, C):
    """<gy, mix(in)> = <mix_vjp(gy), in> for random in, gy, W (the map is linear)."""
    g = np.random.default_rng(30 + L)
    p, off = offsets(L)
    n = 4
    inp = g.standard_normal((n, off[-1], C))
    gy = g.standard_normal((n, (L + 1) ** 2, C))
    W = g.standard_normal(sum(oracle.mix_rows(L)) * C * C)
    lhs = (gy * oracle.channel_mix(L, inp, W)).sum()
    rhs = (oracle.channel_mix_vjp(L, gy, W) * inp).sum()
    assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(lhs))


def test_vjp_identity_blocks_copy_cotangent():
    """W_l = stacked identities: every path block of order l receives gy's block of order l."""
    L, C = 2, 3
    g = np.random.default_rng(9)
    p, off = offsets(L)
    gy = g.standard_normal((5, 9, C))
    W = np.concatenate([np.tile(np.eye(C), (k, 1)).reshape(-1) for k in oracle.mix_rows(L)])
    gin = oracle.channel_mix_vjp(L, gy, W)
    for q, (l1, l2, l3) in enumerate(p):
        np.testing.assert_allclose(gin[:, off[q]:off[q + 1]], gy[:, l3 * l3:(l3 + 1) ** 2], atol=1e-14)


# ------------------------------------------------------- weight gradient

@pytest.mark.parametrize("L,C", [(1, 3), (2, 4), (3, 2), (4, 1)])
def test_wgrad_is_the_gradient_of_the_pairing(L, C):
    """The mixing is linear in W, so <gW, W> = <gy, mix(in, W)> for every W
    (mix from the oracle's forward loops, gW from its weight-gradient loops)."""
    g = np.random.default_rng(40 + L)
    p, off = offsets(L)
    n = 5
    inp = g.standard_normal((n, off[-1], C))
    gy = g.standard_normal((n, (L + 1) ** 2, C))
    gW = oracle.channel_mix_wgrad(L, inp, gy)
    for trial in range(3):
        W = g.standard_normal(sum(oracle.mix_rows(L)) * C * C)
        lhs = (gW * W).sum()
        rhs = (gy * oracle.channel_mix(L, inp, W)).sum()
        assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(rhs))


def test_wgrad_outer_product_of_one_path():
    """One node, one nonzero path block of the input and one nonzero component
    row of gy: gW is that path's block, the outer product in (x) gy, and zero
    elsewhere."""
    L, C = 2, 3
    g = np.random.default_rng(12)
    p, off = offsets(L)
    rows = oracle.mix_rows(L)
    q = 7                                  # a path of order l3
    l3 = int(p[q][2])
    m = 1 if l3 > 0 else 0
    inp = np.zeros((1, off[-1], C))
    a = g.standard_normal(C)
    inp[0, off[q] + m] = a
    gy = np.zeros((1, (L + 1) ** 2, C))
    b = g.standard_normal(C)
    gy[0, l3 * l3 + m] = b
    gW = oracle.channel_mix_wgrad(L, inp, gy)
    rank = int(sum(1 for r in range(q) if p[r][2] == l3))
    start = sum(rows[:l3]) * C * C + rank * C * C
    expect = np.zeros_like(gW)
    expect[start:start + C * C] = np.outer(a, b).reshape(-1)
    np.testing.assert_allclose(gW, expect, atol=1e-15)


def test_wgrad_sums_over_nodes_and_components():
    """gW of a batch = the sum of the per-node gW (a sum over nodes), and a
    mismatched component (gy on another m) contributes nothing."""
    L, C = 3, 2
    g = np.random.default_rng(13)
    p, off = offsets(L)
    inp = g.standard_normal((6, off[-1], C))
    gy = g.standard_normal((6, 16, C))
    whole = oracle.channel_mix_wgrad(L, inp, gy)
    parts = sum(oracle.channel_mix_wgrad(L, inp[i:i + 1], gy[i:i + 1]) for i in range(6))
    np.testing.assert_allclose(whole, parts, rtol=1e-13, atol=1e-13)
