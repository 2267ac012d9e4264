"""Run-to-run bitwise determinism at full size, and the zero-length bond
vector contract, through the C ABI.

Determinism: the kernels use no float atomics and sum in fixed orders, so two
calls on the same inputs give identical bits. Checked where the most orders
meet: l_max = 3 and 4 on the 1024 x 128 graph (several path-group launches
adding into grad_vec / d_vec and into node rows an earlier group stored), the
radial VJP (grad_h, grad_vec through parked per-chunk sums), and one
destination-row chunk of the 32768-atom diamond with its own transpose.

Zero-length vector: the library's documented reading of r = 0 is
Y = (1, 0, ..., 0) with zero derivatives. With that Y only the paths with
l2 = 0 carry a message, and their coefficients are the identity (the
(l, 0 -> l) block), so an edge with r = 0 contributes w[e, p] x[j, l1] to
path p = (l1, 0, l1) and nothing else; every derivative through r is zero.
The test compares against the oracle on the other edges plus that closed
form for the zero edges.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_common import FP32_TOL, dev, rel_err

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def _device_problem(wl, seed=7):
    """Graph + transpose + device-drawn operands (values need not match the
    oracle: only run-to-run equality is checked)."""
    import torch
    from equivariant_interatomic_potentials_amd import etp
    E, n, N, L, C, P = wl.E, wl.n, wl.n_dst, wl.L, wl.C, wl.P
    d = {"plan": etp.etp_plan_create(L, C)}
    rp, src = dev(wl.row_ptr.astype(np.int32)), dev(wl.src.astype(np.int32))
    sp = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    pm = torch.empty(E, dtype=torch.int32, device="cuda")
    pd = torch.empty(E, dtype=torch.int32, device="cuda")
    ws = torch.empty(etp.etp_csr_transpose_workspace(n) // 4 + 1, dtype=torch.int32, device="cuda")
    etp.etp_csr_transpose(etp.Graph(N, n, rp, src), sp, pm, pd, ws)
    d["g"] = etp.Graph(N, n, rp, src, sp, pm, pd)
    d["vec"] = dev(wl.vec.astype(np.float32))
    d["x"] = workloads.device_normal((n, wl.Din, C), seed, "x", 1)
    d["w"] = workloads.device_normal((E, P, C), seed, "w", 1, 1.0 / np.sqrt(P))
    d["G"] = workloads.device_normal((N, wl.Dout, C), seed, "G", 1)
    d["ggx"] = workloads.device_normal((n, wl.Din, C), seed, "ggx", 1)
    d["ggw"] = workloads.device_normal((E, P, C), seed, "ggw", 1)
    d["ggv"] = workloads.device_normal((E, 3), seed, "ggvec", 1)
    return d


def _all_outputs(etp, d, wl):
    import torch
    E, n, N, C, P = wl.E, wl.n, wl.n_dst, wl.C, wl.P
    out = torch.empty(N, wl.Dout, C, device="cuda")
    etp.etp_edge_conv_fwd(d["plan"], d["g"], d["vec"], d["x"], d["w"], out)
    gx, gr = torch.empty(n, wl.Din, C, device="cuda"), torch.empty(E, 3, device="cuda")
    gw = torch.empty(E, P, C, device="cuda")
    etp.etp_edge_conv_vjp(d["plan"], d["g"], d["vec"], d["x"], d["w"], d["G"], gx, gw, gr)
    res = [out, gx, gr, gw.sum(dim=(1, 2)), gw[::97].clone()]
    del gw
    dx, dr, dG = torch.empty_like(gx), torch.empty_like(gr), torch.empty_like(out)
    dw = torch.empty(E, P, C, device="cuda")
    etp.etp_edge_conv_vjp2(d["plan"], d["g"], d["vec"], d["x"], d["w"], d["G"], d["ggx"], d["ggw"], d["ggv"],
                           dx, dw, dr, dG)
    res += [dx, dr, dG, dw.sum(dim=(1, 2)), dw[::97].clone()]
    del dw
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("name", ["micro3", "micro4"])
def test_full_size_run_twice(name):
    import torch
    from equivariant_interatomic_potentials_amd import etp
    say("determinism", name)
    wl = workloads.get(name)
    d = _device_problem(wl)
    a = _all_outputs(etp, d, wl)
    b = _all_outputs(etp, d, wl)
    for k, (u, v) in enumerate(zip(a, b)):
        assert torch.equal(u, v), k


@pytest.mark.parametrize("L,C", [(3, 256), (4, 128)])
def test_radial_vjp_run_twice(L, C):
    """grad_x, grad_h and grad_vec of the radial VJP at several path groups
    (and two 128-channel chunks at C = 256) are identical on a second call."""
    import torch
    from equivariant_interatomic_potentials_amd import etp
    say("determinism radial", L, C)
    row_ptr, src, vec = workloads._micro_graph(0)
    wl = workloads.Workload(f"rad{L}", L, C, 1024, row_ptr, src, vec, 0)
    d = _device_problem(wl)
    K = 8
    h, Wr = workloads.radial_inputs(wl.E, K, L, C, seed=0)
    h, Wr = torch.from_numpy(h).cuda(), torch.from_numpy(Wr).cuda()
    outs = []
    for _ in range(2):
        gx = torch.empty(wl.n, wl.Din, C, device="cuda")
        gh, gr = torch.empty(wl.E, K, device="cuda"), torch.empty(wl.E, 3, device="cuda")
        y = torch.empty(wl.n_dst, wl.Dout, C, device="cuda")
        etp.etp_edge_conv_fwd_radial(d["plan"], d["g"], d["vec"], d["x"], h, Wr, y)
        etp.etp_edge_conv_vjp_radial(d["plan"], d["g"], d["vec"], d["x"], h, Wr, d["G"], gx, gh, gr)
        torch.cuda.synchronize()
        outs.append((y, gx, gh, gr))
    for u, v in zip(*outs):
        assert torch.equal(u, v)


def test_diamond_chunk_run_twice():
    """One destination-row chunk of the 32768-atom diamond (l_max = 3,
    C = 128, about 158 in-edges per row) on its own sub-CSR and transpose."""
    import torch
    from equivariant_interatomic_potentials_amd import etp
    say("determinism diamond chunk")
    full = workloads.get("diamond")
    r0, r1 = 12000, 14048
    e0, e1 = int(full.row_ptr[r0]), int(full.row_ptr[r1])
    wl = workloads.Workload("diamond_chunk", 3, 128, full.n, (full.row_ptr[r0:r1 + 1] - e0).astype(np.int32),
                            full.src[e0:e1], full.vec[e0:e1], 0)
    wl.n_dst = r1 - r0
    d = _device_problem(wl)
    a = _all_outputs(etp, d, wl)
    b = _all_outputs(etp, d, wl)
    for k, (u, v) in enumerate(zip(a, b)):
        assert torch.equal(u, v), k


# ------------------------------------------------- zero-length bond vectors

def test_sh_of_zero_vector():
    import torch
    from equivariant_interatomic_potentials_amd import etp
    say("sh zero vector")
    for L in range(5):
        D = (L + 1) ** 2
        plan = etp.etp_plan_create(L, 8)
        v = torch.zeros(3, 3, device="cuda")
        v[1] = torch.tensor([0.3, -1.2, 2.0])
        Y, dY = torch.empty(3, D, device="cuda"), torch.empty(3, 3, D, device="cuda")
        etp.etp_sh(plan, v, Y, dY)
        Y, dY = Y.cpu().numpy(), dY.cpu().numpy()
        want = np.zeros(D)
        want[0] = 1.0
        for r in (0, 2):
            assert np.array_equal(Y[r], want)
            assert not dY[r].any()
        ry, rdy = oracle.sh(L, np.array([[0.3, -1.2, 2.0]]), grad=True)
        assert rel_err(Y[1], ry[0]) < FP32_TOL and rel_err(dY[1], rdy[0]) < FP32_TOL


def _zero_edge_closed_forms(wl, zero, x, w, G, Xp, Wp):
    """Contributions of the zero-vector edges (Y = (1, 0, ...), dY = 0) by the
    identity coupling of the paths (l1, 0, l1): out, gx, gw, dG, dx, dw."""
    Ps = oracle.paths(wl.L)
    off = np.concatenate([[0], np.cumsum(2 * Ps[:, 2] + 1)])
    dst = np.repeat(np.arange(wl.n_dst), np.diff(wl.row_ptr))
    out = np.zeros((wl.n_dst, wl.Dout, wl.C))
    gx = np.zeros((wl.n, wl.Din, wl.C))
    gw = np.zeros((wl.E, wl.P, wl.C))
    dG = np.zeros_like(out)
    dx = np.zeros_like(gx)
    dw = np.zeros_like(gw)
    for e in np.nonzero(zero)[0]:
        i, j = dst[e], wl.src[e]
        for p, (l1, l2, l3) in enumerate(Ps):
            if l2 != 0:
                continue
            xr = slice(l1 * l1, (l1 + 1) ** 2)
            orow = slice(off[p], off[p + 1])
            out[i, orow] += w[e, p] * x[j, xr]
            gx[j, xr] += w[e, p] * G[i, orow]
            gw[e, p] = (x[j, xr] * G[i, orow]).sum(axis=0)
            dG[i, orow] += w[e, p] * Xp[j, xr] + Wp[e, p] * x[j, xr]
            dx[j, xr] += Wp[e, p] * G[i, orow]
            dw[e, p] = (Xp[j, xr] * G[i, orow]).sum(axis=0)
    return out, gx, gw, dG, dx, dw


@pytest.mark.parametrize("L,C", [(1, 8), (2, 128), (3, 64)])
def test_zero_length_bond_vectors(L, C):
    """Edges with r = 0 among ordinary ones: forward, VJP and VJP-of-VJP
    against the oracle on the ordinary edges plus the closed form of the
    zero edges; grad_vec and d_vec of a zero edge are exactly 0."""
    import torch
    from gpu_common import DeviceProblem, np_
    say("zero vectors", L, C)
    wl = workloads.small(L, C, 40, 12, seed=50 + L, empty_rows=False)
    zero = np.zeros(wl.E, bool)
    zero[np.random.default_rng(L).choice(wl.E, max(3, wl.E // 8), replace=False)] = True
    vec = wl.vec.copy()
    vec[zero] = 0.0
    wl.vec = vec
    p = DeviceProblem(wl)
    out = np_(p.fwd())
    gx, gw, gr = (np_(t) for t in p.vjp())
    dx, dw, dr, dG = (np_(t) for t in p.vjp2())
    torch.cuda.synchronize()
    # the oracle on the ordinary edges (zero edges' weights and cotangents set to 0)
    keep = (~zero)[:, None, None]
    w_nz, ggw_nz = wl.w * keep, wl.ggw * keep
    vec_safe = vec.copy()
    vec_safe[zero] = (1.0, 0.0, 0.0)  # any direction: its weights are 0
    ref_out = oracle.fwd(L, wl.row_ptr, wl.src, vec_safe, wl.x, w_nz)
    rgx, rgw, rgr = oracle.vjp(L, wl.row_ptr, wl.src, vec_safe, wl.x, w_nz, wl.G)
    ggv = wl.ggvec.copy()
    ggv[zero] = 0.0
    rdx, rdw, rdr, rdG = oracle.vjp2(L, wl.row_ptr, wl.src, vec_safe, wl.x, w_nz, wl.G, wl.ggx, ggw_nz, ggv)
    zo, zgx, zgw, zdG, zdx, zdw = _zero_edge_closed_forms(wl, zero, wl.x.astype(np.float64),
                                                         wl.w.astype(np.float64), wl.G.astype(np.float64),
                                                         wl.ggx.astype(np.float64), wl.ggw.astype(np.float64))
    assert rel_err(out, ref_out + zo) < FP32_TOL
    assert rel_err(gx, rgx + zgx) < FP32_TOL
    rgw = np.where(keep, rgw, zgw)
    assert rel_err(gw, rgw) < FP32_TOL
    assert not gr[zero].any() and not dr[zero].any()
    assert rel_err(gr[~zero], rgr[~zero]) < FP32_TOL
    assert rel_err(dG, rdG + zdG) < FP32_TOL
    assert rel_err(dx, rdx + zdx) < FP32_TOL
    assert rel_err(dw, np.where(keep, rdw, zdw)) < FP32_TOL
    assert rel_err(dr[~zero], rdr[~zero]) < FP32_TOL
