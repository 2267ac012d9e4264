"""Pins for the oracle's periodic neighbour list (float32 decision, minimum
image, strict cutoff, rows sorted by source).

  * exact lattice: positions on a 1/8 grid in a box of 8, where every float32
    step is exact, against integer brute force (minimum image by integer
    remainders, squared distance compared in integers);
  * agreement with scipy's periodic k-d tree (an independent float64
    implementation) on the water box, up to pairs within rounding of the
    cutoff;
  * worked cases: a pair across the boundary (value and sign of the
    minimum-image vector), a pair at exactly the cutoff (excluded) and one
    ulp inside it (included), self pairs excluded;
  * exact antisymmetry of the list and its vectors; invariance under whole-box
    translations on the exact lattice.
"""
import numpy as np

import oracle
import workloads


def _lattice_case(seed, n, box_units=64, rc_units=20):
    """Positions on a grid of spacing 1/8 (box 8, rc 2.5): exact in float32."""
    g = np.random.default_rng(seed)
    ip = g.integers(-3 * box_units, 4 * box_units, size=(n, 3))
    return ip, ip.astype(np.float32) / 8.0, box_units / 8.0, rc_units / 8.0


def _int_brute(ip, box_units, rc_units):
    n = ip.shape[0]
    rows = []
    for i in range(n):
        row = []
        for j in range(n):
            if j == i:
                continue
            d = (ip[j] - ip[i]) % box_units
            d = np.where(d > box_units // 2, d - box_units, d)
            # a component of exactly half the box: rint(0.5) = 0 keeps +half,
            # rint(-0.5) = -0 keeps -half; either image has the same length
            if int((d * d).sum()) < rc_units * rc_units:
                row.append(j)
        rows.append(row)
    return rows


def _rows(row_ptr, src):
    return [list(src[row_ptr[i]:row_ptr[i + 1]]) for i in range(len(row_ptr) - 1)]


def test_exact_lattice_matches_integer_brute_force():
    for seed, n in [(0, 60), (1, 150), (2, 7)]:
        ip, pos, box, rc = _lattice_case(seed, n)
        row_ptr, src, vec = oracle.neighbors(pos, box, rc)
        want = _int_brute(ip, 64, 20)
        assert _rows(row_ptr, src) == want
        # vectors: the integer minimum image, scaled
        dst = np.repeat(np.arange(n), np.diff(row_ptr))
        d = (ip[src] - ip[dst]) % 64
        d = np.where(d > 32, d - 64, d)
        d = np.where(d == 32, np.sign(vec) * 32, d)  # half-box components: either sign
        np.testing.assert_array_equal(vec, d.astype(np.float32) / 8.0)


def test_lattice_whole_box_translation_invariance():
    ip, pos, box, rc = _lattice_case(3, 120)
    ref = oracle.neighbors(pos, box, rc)
    shift = np.array([box, -2 * box, 5 * box], np.float32)
    got = oracle.neighbors(pos + shift, box, rc)
    np.testing.assert_array_equal(ref[0], got[0])
    np.testing.assert_array_equal(ref[1], got[1])
    np.testing.assert_array_equal(ref[2], got[2])


def test_agrees_with_periodic_kd_tree_on_water():
    pos, box = workloads.water_positions(0)
    rc = 6.0
    row_ptr, src, vec = oracle.neighbors(pos, box, rc)
    kd_ptr, kd_src, kd_vec = workloads.cutoff_csr(pos, box, rc)
    n = pos.shape[0]
    dst = np.repeat(np.arange(n), np.diff(row_ptr))
    kd_dst = np.repeat(np.arange(n), np.diff(kd_ptr))
    a = set(zip(dst.tolist(), src.tolist()))
    b = set(zip(kd_dst.tolist(), kd_src.tolist()))
    p = np.mod(pos, box)
    for i, j in a ^ b:  # only pairs within float32 rounding of the cutoff may differ
        d = p[j] - p[i]
        d -= box * np.round(d / box)
        assert abs(np.linalg.norm(d) - rc) < 1e-5
    assert len(a ^ b) <= 4
    if not (a ^ b):
        np.testing.assert_array_equal(row_ptr, kd_ptr)
        np.testing.assert_array_equal(src, kd_src)
        np.testing.assert_allclose(vec, kd_vec, atol=2e-5, rtol=0)
    # sorted rows, no self pairs
    assert np.all(dst != src)
    for i in range(0, n, 97):
        r = src[row_ptr[i]:row_ptr[i + 1]]
        assert np.all(np.diff(r) > 0)


def test_worked_cases():
    # across the boundary: the minimum image of 9.7 seen from 0.5 in a box of 10 is -0.3
    pos = np.array([[0.5, 5.0, 5.0], [9.7, 5.0, 5.0]], np.float32)
    row_ptr, src, vec = oracle.neighbors(pos, 10.0, 1.0)
    np.testing.assert_array_equal(row_ptr, [0, 1, 2])
    np.testing.assert_array_equal(src, [1, 0])
    np.testing.assert_allclose(vec[0], [-0.8, 0, 0], atol=1e-6)
    np.testing.assert_allclose(vec[1], [0.8, 0, 0], atol=1e-6)
    # exactly at the cutoff: not a neighbour; one ulp inside: a neighbour
    pos = np.array([[1.0, 1.0, 1.0], [3.0, 1.0, 1.0]], np.float32)
    assert oracle.neighbors(pos, 10.0, 2.0)[0][-1] == 0
    rc_up = np.nextafter(np.float32(2.0), np.float32(3.0))
    assert oracle.neighbors(pos, 10.0, rc_up)[0][-1] == 2
    # coincident atoms are neighbours of each other (distance 0), never of themselves
    pos = np.array([[2.0, 2.0, 2.0], [2.0, 2.0, 2.0], [7.0, 7.0, 7.0]], np.float32)
    row_ptr, src, vec = oracle.neighbors(pos, 10.0, 1.0)
    np.testing.assert_array_equal(row_ptr, [0, 1, 2, 2])
    np.testing.assert_array_equal(src, [1, 0])
    assert not vec.any()
    # no atoms
    row_ptr, src, vec = oracle.neighbors(np.zeros((0, 3), np.float32), 10.0, 1.0)
    np.testing.assert_array_equal(row_ptr, [0])
    assert src.size == 0


def test_antisymmetric():
    g = np.random.default_rng(7)
    box = np.array([9.0, 11.5, 10.25], np.float32)
    pos = (g.random((300, 3)) * box * 3 - box).astype(np.float32)
    row_ptr, src, vec = oracle.neighbors(pos, box, 3.0)
    n = pos.shape[0]
    dst = np.repeat(np.arange(n), np.diff(row_ptr))
    edges = {(i, j): v for i, j, v in zip(dst.tolist(), src.tolist(), vec)}
    assert len(edges) == len(src) > 0
    for (i, j), v in edges.items():
        np.testing.assert_array_equal(edges[(j, i)], -v)
