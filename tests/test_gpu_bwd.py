"""GPU parity of the destination-side backward (etp_edge_conv_vjp_ws and
etp_edge_conv_vjp2_ws, through the C ABI) against the float64 oracle.

Same bar as the other parity tests: per output tensor max |gpu - oracle| /
max |oracle| <= 1e-5 with fp32 features, <= 1e-2 with bf16-stored features
against the oracle fed the unrounded values (and <= 1e-5 against the oracle
fed the rounded ones). The cases mirror the source-side VJP's: ragged rows
with empty ones, long destination and source segments, channel counts that
leave a chunk partly filled (and a node block whose float count is not a
multiple of four), several path groups at l_max = 3 and 4, null outputs and
cotangents, accumulation, a graph without edges, the full-size workloads on
sampled rows, and run-to-run bitwise equality.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_common import BF16_TOL, FP32_TOL, DeviceProblem, dev, dst_subgraph, np_, rel_err, src_subgraph

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def small_wl(L, C, kind):
    if kind == "ragged":
        return workloads.small(L, C, 23, 14, seed=L * 100 + C)
    if kind == "fan_in":
        return workloads.bipartite(L, C, 5, 400, 250, 390, seed=L + C)
    return workloads.bipartite(L, C, 300, 6, 1, 6, seed=L + 7 * C)


# the destination-side formulation is forced here (the calls would pick the
# source side for some shapes); the default choice is checked separately
FORCE = 4  # ETP_FLAG_DST_PASS


def vjp_ws(p, want=("gx", "gw", "gr"), flags=FORCE, gx=None, ws=True):
    wl, etp = p.wl, p.etp
    if gx is None and "gx" in want:
        gx = p.empty(wl.n, wl.Din, wl.C)
    gw = p.empty(wl.E, wl.P, wl.C) if "gw" in want else None
    gr = p.empty(wl.E, 3) if "gr" in want else None
    w = etp.bwd_workspace(p.plan, p.graph) if ws else None
    etp.etp_edge_conv_vjp_ws(p.plan, p.graph, p.vec, p.x, p.w, p.G, gx, gw, gr, w, flags)
    return gx, gw, gr


def vjp2_ws(p, cot=("ggx", "ggw", "ggvec"), want=("dx", "dw", "dr", "dG"), flags=FORCE, dx=None, dG=None,
            ws=True):
    wl, etp = p.wl, p.etp
    ggx = dev(wl.ggx) if "ggx" in cot else None
    ggw = dev(wl.ggw) if "ggw" in cot else None
    ggv = dev(wl.ggvec) if "ggvec" in cot else None
    if dx is None and "dx" in want:
        dx = p.empty(wl.n, wl.Din, wl.C)
    dw = p.empty(wl.E, wl.P, wl.C) if "dw" in want else None
    dr = p.empty(wl.E, 3) if "dr" in want else None
    if dG is None and "dG" in want:
        dG = p.empty(wl.n_dst, wl.Dout, wl.C)
    w = etp.bwd_workspace(p.plan, p.graph, etp.ETP_OP_VJP2_WS) if ws else None
    etp.etp_edge_conv_vjp2_ws(p.plan, p.graph, p.vec, p.x, p.w, p.G, ggx, ggw, ggv, dx, dw, dr, dG, w, flags)
    return dx, dw, dr, dG


SMALL = [
    (0, 8, "ragged"), (1, 8, "ragged"), (1, 5, "ragged"), (2, 8, "ragged"), (2, 64, "ragged"),
    (2, 96, "ragged"), (2, 128, "ragged"), (3, 16, "ragged"), (3, 128, "ragged"), (4, 8, "ragged"),
    (4, 128, "ragged"),
    (2, 128, "fan_in"), (2, 64, "fan_out"), (3, 128, "fan_in"), (4, 64, "fan_out"), (1, 8, "fan_out"),
    (2, 200, "ragged"), (1, 256, "fan_out"), (2, 1, "ragged"), (4, 1, "ragged"), (3, 256, "ragged"),
    (2, 6, "ragged"), (4, 10, "fan_in"),
]


@pytest.mark.parametrize("L,C,kind", SMALL)
def test_vjp_ws_small(L, C, kind):
    say("vjp_ws", L, C, kind)
    wl = small_wl(L, C, kind)
    p = DeviceProblem(wl)
    gx, gw, gr = (np_(t) for t in vjp_ws(p))
    rgx, rgw, rgr = oracle.vjp(L, wl.row_ptr, wl.src, wl.vec, wl.x, wl.w, wl.G)
    assert rel_err(gx, rgx) < FP32_TOL, rel_err(gx, rgx)
    assert rel_err(gw, rgw) < FP32_TOL, rel_err(gw, rgw)
    assert rel_err(gr, rgr) < FP32_TOL, rel_err(gr, rgr)


@pytest.mark.parametrize("L,C,kind", SMALL)
def test_vjp2_ws_small(L, C, kind):
    say("vjp2_ws", L, C, kind)
    wl = small_wl(L, C, kind)
    p = DeviceProblem(wl)
    got = [np_(t) for t in vjp2_ws(p)]
    r = oracle.vjp2(L, wl.row_ptr, wl.src, wl.vec, wl.x, wl.w, wl.G, wl.ggx, wl.ggw, wl.ggvec)
    for name, g_, ref in zip(("dx", "dw", "dr", "dG"), got, r):
        assert rel_err(g_, ref) < FP32_TOL, (name, rel_err(g_, ref))


@pytest.mark.parametrize("cot", [("ggx",), ("ggw",), ("ggvec",), ("ggx", "ggw"), ()])
def test_vjp2_ws_null_cotangents(cot):
    L, C = 3, 64
    say("vjp2_ws-null", cot)
    wl = small_wl(L, C, "ragged")
    p = DeviceProblem(wl)
    got = [np_(t) for t in vjp2_ws(p, cot=cot)]
    r = oracle.vjp2(L, wl.row_ptr, wl.src, wl.vec, wl.x, wl.w, wl.G,
                    wl.ggx if "ggx" in cot else None, wl.ggw if "ggw" in cot else None,
                    wl.ggvec if "ggvec" in cot else None)
    for name, g_, ref in zip(("dx", "dw", "dr", "dG"), got, r):
        if np.abs(ref).max() == 0:
            assert np.abs(g_).max() == 0, name
        else:
            assert rel_err(g_, ref) < FP32_TOL, (name, rel_err(g_, ref))


def test_ws_null_outputs_and_accumulate():
    import torch
    from equivariant_interatomic_potentials_amd import etp
    L, C = 3, 128
    say("ws null-outputs/accumulate")
    wl = small_wl(L, C, "ragged")
    p = DeviceProblem(wl)
    gx, gw, gr = vjp_ws(p)
    _, _, gr2 = vjp_ws(p, want=("gr",), ws=False)      # no node gradient: no workspace needed
    assert torch.equal(gr, gr2)
    _, gw3, _ = vjp_ws(p, want=("gw",), ws=False)
    assert torch.equal(gw, gw3)
    gx4 = gx.clone()
    vjp_ws(p, want=("gx",), flags=etp.ETP_FLAG_ACCUMULATE | FORCE, gx=gx4)
    assert rel_err(np_(gx4), 2 * np_(gx)) < FP32_TOL
    dx, dw, dr, dG = vjp2_ws(p)
    _, dw2, _, _ = vjp2_ws(p, want=("dw",))
    assert torch.equal(dw, dw2)
    _, _, _, dG2 = vjp2_ws(p, want=("dG",))
    assert torch.equal(dG, dG2)
    dx3, dG3 = dx.clone(), dG.clone()
    vjp2_ws(p, want=("dx", "dG"), flags=etp.ETP_FLAG_ACCUMULATE | FORCE, dx=dx3, dG=dG3)
    assert rel_err(np_(dx3), 2 * np_(dx)) < FP32_TOL
    assert rel_err(np_(dG3), 2 * np_(dG)) < FP32_TOL


def test_ws_workspace_checks():
    """grad_x without a (large enough) workspace is refused before any launch."""
    import torch
    from equivariant_interatomic_potentials_amd import etp
    say("ws checks")
    wl = small_wl(2, 8, "ragged")
    p = DeviceProblem(wl)
    gx = p.empty(wl.n, wl.Din, wl.C)
    need = etp.etp_workspace_size(p.plan, etp.ETP_OP_VJP_WS, p.graph)
    assert need == wl.E * (wl.Din * wl.C + 6) * 4
    assert etp.etp_workspace_size(p.plan, etp.ETP_OP_VJP2_WS, p.graph) == need
    small = torch.empty(need - 4, dtype=torch.uint8, device="cuda")
    for ws in (None, small):
        with pytest.raises(etp.EtpError) as ei:
            etp.etp_edge_conv_vjp_ws(p.plan, p.graph, p.vec, p.x, p.w, p.G, gx, None, None, ws, FORCE)
        assert ei.value.status == etp.ETP_ERR_WORKSPACE
    big = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(etp.EtpError) as ei:  # misaligned
        etp.etp_edge_conv_vjp_ws(p.plan, p.graph, p.vec, p.x, p.w, p.G, gx, None, None, big[4:4 + need], FORCE)
    assert ei.value.status == etp.ETP_ERR_WORKSPACE
    torch.cuda.synchronize()


def test_ws_empty_graph_zeroes_node_outputs():
    import torch
    from equivariant_interatomic_potentials_amd import etp
    say("ws empty-graph")
    wl = workloads.small(3, 64, 7, 0, seed=5)
    assert wl.E == 0
    p = DeviceProblem(wl)
    gx = torch.full((wl.n, wl.Din, wl.C), 7.0, device="cuda")
    vjp_ws(p, want=("gx",), gx=gx, ws=False)
    assert float(gx.abs().max()) == 0.0
    dx = torch.full((wl.n, wl.Din, wl.C), 7.0, device="cuda")
    dG = torch.full((wl.n_dst, wl.Dout, wl.C), 7.0, device="cuda")
    vjp2_ws(p, want=("dx", "dG"), dx=dx, dG=dG)
    assert float(dx.abs().max()) == 0.0 and float(dG.abs().max()) == 0.0


@pytest.mark.parametrize("L,C", [(1, 8), (2, 128), (3, 128)])
def test_ws_bf16_features(L, C):
    say("ws bf16", L, C)
    wl = small_wl(L, C, "ragged")
    p = DeviceProblem(wl, bf16=True)
    gx, gw, gr = (np_(t) for t in vjp_ws(p))
    dx, dw, dr, dG = (np_(t) for t in vjp2_ws(p))
    got = dict(gx=gx, gw=gw, gr=gr, dx=dx, dw=dw, dr=dr, dG=dG)
    for xin, tol in ((p.x_seen, FP32_TOL), (wl.x, BF16_TOL)):
        ref = dict(zip(("gx", "gw", "gr"), oracle.vjp(L, wl.row_ptr, wl.src, wl.vec, xin, wl.w, wl.G)))
        ref.update(zip(("dx", "dw", "dr", "dG"),
                       oracle.vjp2(L, wl.row_ptr, wl.src, wl.vec, xin, wl.w, wl.G, wl.ggx, wl.ggw, wl.ggvec)))
        for k in got:
            assert rel_err(got[k], ref[k]) < tol, (k, tol, rel_err(got[k], ref[k]))


@pytest.mark.parametrize("name", ["micro", "micro3", "micro4", "water"])
def test_ws_full_config_sampled(name):
    """The benchmarked shapes at full size, sampled rows against the oracle,
    and a second call bit for bit equal to the first."""
    import torch
    say("ws full", name)
    wl = workloads.get(name)
    p = DeviceProblem(wl)
    L = wl.L
    g = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, wl.n_dst - 1], g.choice(wl.n_dst, 5, replace=False)]))
    cols = np.unique(np.concatenate([[0, wl.n - 1], g.choice(wl.n, 5, replace=False)]))
    rp, eidx = dst_subgraph(wl, rows)
    rp2, eidx2 = src_subgraph(wl, cols)

    gx, gw, gr = vjp_ws(p)
    rgx, rgw, rgr = oracle.vjp(L, rp2, wl.src[eidx2], wl.vec[eidx2], wl.x, wl.w[eidx2], wl.G)
    assert rel_err(np_(gx)[cols], rgx[cols]) < FP32_TOL
    assert rel_err(np_(gw)[eidx2], rgw) < FP32_TOL
    assert rel_err(np_(gr)[eidx2], rgr) < FP32_TOL
    gx2, gw2, gr2 = vjp_ws(p)
    assert torch.equal(gx, gx2) and torch.equal(gw, gw2) and torch.equal(gr, gr2)
    del gx, gw, gr, gx2, gw2, gr2

    dx, dw, dr, dG = vjp2_ws(p)
    r_dst = oracle.vjp2(L, rp, wl.src[eidx], wl.vec[eidx], wl.x, wl.w[eidx], wl.G[rows], wl.ggx,
                        wl.ggw[eidx], wl.ggvec[eidx])
    assert rel_err(np_(dG)[rows], r_dst[3]) < FP32_TOL
    r_src = oracle.vjp2(L, rp2, wl.src[eidx2], wl.vec[eidx2], wl.x, wl.w[eidx2], wl.G, wl.ggx,
                        wl.ggw[eidx2], wl.ggvec[eidx2])
    assert rel_err(np_(dx)[cols], r_src[0][cols]) < FP32_TOL
    assert rel_err(np_(dw)[eidx2], r_src[1]) < FP32_TOL
    assert rel_err(np_(dr)[eidx2], r_src[2]) < FP32_TOL
    dx2, dw2, dr2, dG2 = vjp2_ws(p)
    for u, v in ((dx, dx2), (dw, dw2), (dr, dr2), (dG, dG2)):
        assert torch.equal(u, v)


@pytest.mark.parametrize("L,C", [(1, 8), (2, 64), (2, 128), (3, 128), (4, 64)])
def test_ws_default_and_forced_formulations(L, C):
    """Without a forcing flag the calls pick a formulation per shape; each
    choice, and each forced one, matches the oracle, and forcing both is
    refused."""
    import torch
    from equivariant_interatomic_potentials_amd import etp
    say("ws default", L, C)
    wl = small_wl(L, C, "ragged")
    p = DeviceProblem(wl)
    ref = oracle.vjp(L, wl.row_ptr, wl.src, wl.vec, wl.x, wl.w, wl.G)
    ref2 = oracle.vjp2(L, wl.row_ptr, wl.src, wl.vec, wl.x, wl.w, wl.G, wl.ggx, wl.ggw, wl.ggvec)
    for f in (0, etp.ETP_FLAG_SRC_PASS, etp.ETP_FLAG_DST_PASS):
        got = [np_(t) for t in vjp_ws(p, flags=f)]
        for a, b in zip(got, ref):
            assert rel_err(a, b) < FP32_TOL
        got = [np_(t) for t in vjp2_ws(p, flags=f)]
        for a, b in zip(got, ref2):
            assert rel_err(a, b) < FP32_TOL
    with pytest.raises(etp.EtpError) as ei:
        vjp_ws(p, flags=etp.ETP_FLAG_SRC_PASS | etp.ETP_FLAG_DST_PASS)
    assert ei.value.status == etp.ETP_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()


@pytest.mark.parametrize("L,C,kind", [(3, 128, "ragged"), (3, 64, "fan_in"), (3, 16, "fan_out")])
def test_ws_groups_in_one_launch_match_in_sequence(L, C, kind):
    """With a workspace the l_max = 3 path groups run in one launch and their
    bond-vector partials are added in group order afterwards; without one
    (no node gradient wanted) they run one launch after another, each adding
    to the last. Both give the same gr / dr bit for bit, and the same gw / dw."""
    import torch
    say("ws groups one launch vs sequence", L, C, kind)
    p = DeviceProblem(small_wl(L, C, kind))
    _, gw1, gr1 = vjp_ws(p, want=("gw", "gr"), ws=True)
    _, gw2, gr2 = vjp_ws(p, want=("gw", "gr"), ws=False)
    assert torch.equal(gr1, gr2) and torch.equal(gw1, gw2)
    _, dw1, dr1, _ = vjp2_ws(p, want=("dw", "dr"), ws=True)
    _, dw2, dr2, _ = vjp2_ws(p, want=("dw", "dr"), ws=False)
    assert torch.equal(dr1, dr2) and torch.equal(dw1, dw2)
    wl = p.wl
    gx, gw, gr = vjp_ws(p)
    ref = oracle.vjp(L, wl.row_ptr, wl.src, wl.vec, wl.x, wl.w, wl.G)
    for got, exp in zip((gx, gw, gr), ref):
        assert rel_err(np_(got), exp) < FP32_TOL
