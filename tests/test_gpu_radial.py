"""GPU parity of the forward with radial weights formed in the kernel
(w = h Wr, then the convolution) and of its VJP (grad_x, grad_h, grad_vec),
through the C ABI, against the float64 oracle: every l_max, ragged channel
counts (one to four 64-channel chunks), 1..8 basis functions, bf16 features,
accumulate, null outputs, empty rows, the argument checks and the
benchmarked 1024-node microbenchmark at full size on sampled rows."""
import sys

import numpy as np
import pytest

import oracle
import workloads

from gpu_common import BF16_TOL, FP32_TOL, DeviceProblem, dev, dst_subgraph, np_, rel_err, src_subgraph

pytestmark = pytest.mark.gpu


def say(*a):
    print("[radial]", *a, file=sys.stderr, flush=True)


def run(p, h, Wr, flags=0, out=None):
    wl = p.wl
    if out is None:
        out = p.empty(wl.n_dst, wl.Dout, wl.C)
    p.etp.etp_edge_conv_fwd_radial(p.plan, p.graph, p.vec, p.x, dev(h), dev(Wr), out, flags)
    return out


CASES = [(0, 64, 8), (1, 64, 3), (2, 128, 8), (2, 100, 1), (2, 1, 5), (3, 128, 8), (3, 200, 7),
         (4, 64, 8), (4, 130, 2)]


@pytest.mark.parametrize("L,C,K", CASES)
def test_radial_fwd_small(L, C, K):
    say("small", L, C, K)
    wl = workloads.small(L, C, 23, 14, seed=L * 10 + C + K)
    h, Wr = workloads.radial_inputs(wl.E, K, L, C, seed=K)
    p = DeviceProblem(wl, need=())
    out = np_(run(p, h, Wr))
    ref = oracle.fwd_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr)
    assert rel_err(out, ref) < FP32_TOL, rel_err(out, ref)


@pytest.mark.parametrize("L,C", [(2, 128), (3, 64)])
def test_radial_fwd_bf16_features(L, C):
    say("bf16", L, C)
    wl = workloads.small(L, C, 19, 12, seed=5 + L)
    h, Wr = workloads.radial_inputs(wl.E, 8, L, C, seed=3)
    p = DeviceProblem(wl, bf16=True, need=())
    out = np_(run(p, h, Wr))
    ref = oracle.fwd_radial(L, wl.row_ptr, wl.src, wl.vec, p.x_seen, h, Wr)
    assert rel_err(out, ref) < FP32_TOL, rel_err(out, ref)
    ref32 = oracle.fwd_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr)
    assert rel_err(out, ref32) < BF16_TOL


@pytest.mark.parametrize("L,C", [(1, 512), (2, 1024)])
def test_radial_fwd_wide_channels(L, C):
    """The forward's channel chunks go up to 1024 channels (16 workgroups per node)."""
    say("wide", L, C)
    wl = workloads.small(L, C, 11, 6, seed=C + L)
    h, Wr = workloads.radial_inputs(wl.E, 8, L, C, seed=9)
    p = DeviceProblem(wl, need=())
    out = np_(run(p, h, Wr))
    ref = oracle.fwd_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr)
    assert rel_err(out, ref) < FP32_TOL, rel_err(out, ref)


def test_radial_empty_graph():
    """No edges: the forward writes zeros and the VJP zero grad_x."""
    import torch
    say("empty")
    wl = workloads.small(2, 64, 7, 0, seed=5)
    assert wl.E == 0
    h, Wr = workloads.radial_inputs(0, 4, 2, 64, seed=1)
    p = DeviceProblem(wl, need=("G",))
    out = torch.full((wl.n_dst, wl.Dout, wl.C), 7.0, device="cuda")
    run(p, h, Wr, out=out)
    assert float(out.abs().max()) == 0.0
    gx = torch.full((wl.n, wl.Din, wl.C), 7.0, device="cuda")
    run_vjp(p, h, Wr, gx=gx)
    assert float(gx.abs().max()) == 0.0


def test_radial_accumulate_and_empty_rows():
    """ACCUMULATE adds to out; destinations without edges get 0 (or keep out)."""
    import torch
    say("accumulate")
    wl = workloads.bipartite(2, 64, 40, 30, 0, 5, seed=4)
    h, Wr = workloads.radial_inputs(wl.E, 4, 2, 64, seed=4)
    p = DeviceProblem(wl, need=())
    ref = oracle.fwd_radial(2, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr)
    base = torch.randn(wl.n_dst, wl.Dout, wl.C, device="cuda")
    got = run(p, h, Wr, flags=p.etp.ETP_FLAG_ACCUMULATE, out=base.clone())
    assert rel_err(np_(got) - np_(base), ref) < FP32_TOL
    out = run(p, h, Wr, out=torch.full_like(base, 7.0))
    assert rel_err(np_(out), ref) < FP32_TOL
    empty = np.diff(wl.row_ptr) == 0
    assert empty.any() and np.abs(np_(out)[empty]).max() == 0.0


def test_radial_argument_checks():
    import torch
    say("args")
    wl = workloads.small(1, 8, 6, 3, seed=2)
    p = DeviceProblem(wl, need=())
    out = p.empty(wl.n_dst, wl.Dout, wl.C)
    for K in (0, 9):
        h = torch.zeros(wl.E, max(K, 1), device="cuda")
        Wr = torch.zeros(max(K, 1), p.plan.P, wl.C, device="cuda")
        with pytest.raises(p.etp.EtpError) as ei:
            p.etp.etp_edge_conv_fwd_radial(p.plan, p.graph, p.vec, p.x, h if K else None,
                                           Wr if K else None, out)
        assert ei.value.status in (p.etp.ETP_ERR_UNSUPPORTED, p.etp.ETP_ERR_INVALID_ARGUMENT)


def test_radial_micro_full_size_sampled():
    """The 1024-node x 128-neighbour microbenchmark with 8 basis functions,
    in the launch configuration the benchmark times; destination rows
    sampled and recomputed by the oracle."""
    say("micro")
    wl = workloads.get("micro")
    K = 8
    h, Wr = workloads.radial_inputs(wl.E, K, wl.L, wl.C, seed=11)
    p = DeviceProblem(wl, need=())
    out = np_(run(p, h, Wr))
    g = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, wl.n_dst - 1], g.choice(wl.n_dst, 6, replace=False)]))
    rp, eidx = dst_subgraph(wl, rows)
    ref = oracle.fwd_radial(wl.L, rp, wl.src[eidx], wl.vec[eidx], wl.x, h[eidx], Wr)
    assert rel_err(out[rows], ref) < FP32_TOL, rel_err(out[rows], ref)


def run_vjp(p, h, Wr, want=("gx", "gh", "gr"), flags=0, gx=None):
    wl = p.wl
    K = h.shape[1]
    if gx is None and "gx" in want:
        gx = p.empty(wl.n, wl.Din, wl.C)
    gh = p.empty(wl.E, K) if "gh" in want else None
    gr = p.empty(wl.E, 3) if "gr" in want else None
    p.etp.etp_edge_conv_vjp_radial(p.plan, p.graph, p.vec, p.x, dev(h), dev(Wr), p.G, gx, gh, gr, flags)
    return gx, gh, gr


VJP_CASES = [(0, 64, 8), (1, 1, 3), (1, 64, 4), (2, 128, 8), (2, 100, 1), (2, 200, 6), (2, 256, 8),
             (3, 128, 8), (3, 64, 5), (4, 64, 8), (4, 130, 2)]


@pytest.mark.parametrize("L,C,K", VJP_CASES)
def test_radial_vjp_small(L, C, K):
    say("vjp", L, C, K)
    wl = workloads.small(L, C, 23, 14, seed=L * 7 + C + K)
    h, Wr = workloads.radial_inputs(wl.E, K, L, C, seed=K + 1)
    p = DeviceProblem(wl, need=("G",))
    gx, gh, gr = (np_(t) for t in run_vjp(p, h, Wr))
    rgx, rgh, rgr, _ = oracle.vjp_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr, wl.G)
    assert rel_err(gx, rgx) < FP32_TOL, rel_err(gx, rgx)
    assert rel_err(gh, rgh) < FP32_TOL, rel_err(gh, rgh)
    assert rel_err(gr, rgr) < FP32_TOL, rel_err(gr, rgr)


@pytest.mark.parametrize("want", [("gh",), ("gr",), ("gx",), ("gh", "gr")])
def test_radial_vjp_null_outputs(want):
    say("vjp-null", want)
    L, C, K = 2, 128, 8
    wl = workloads.small(L, C, 17, 10, seed=31)
    h, Wr = workloads.radial_inputs(wl.E, K, L, C, seed=2)
    p = DeviceProblem(wl, need=("G",))
    got = dict(zip(("gx", "gh", "gr"), run_vjp(p, h, Wr, want=want)))
    ref = dict(zip(("gx", "gh", "gr"), oracle.vjp_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr, wl.G)))
    for k in want:
        assert rel_err(np_(got[k]), ref[k]) < FP32_TOL, (k, rel_err(np_(got[k]), ref[k]))


def test_radial_vjp_accumulate_and_fan_out():
    """ACCUMULATE adds grad_x; few sources with many out-edges each, then many
    sources per destination."""
    import torch
    say("vjp-acc")
    L, C, K = 2, 64, 4
    wl = workloads.bipartite(L, C, 300, 6, 1, 6, seed=8)
    h, Wr = workloads.radial_inputs(wl.E, K, L, C, seed=5)
    p = DeviceProblem(wl, need=("G",))
    rgx, rgh, rgr, _ = oracle.vjp_radial(L, wl.row_ptr, wl.src, wl.vec, wl.x, h, Wr, wl.G)
    base = torch.randn(wl.n, wl.Din, wl.C, device="cuda")
    gx, gh, gr = run_vjp(p, h, Wr, flags=p.etp.ETP_FLAG_ACCUMULATE, gx=base.clone())
    assert rel_err(np_(gx) - np_(base), rgx) < FP32_TOL
    assert rel_err(np_(gh), rgh) < FP32_TOL
    assert rel_err(np_(gr), rgr) < FP32_TOL
    wl2 = workloads.bipartite(L, C, 5, 400, 250, 390, seed=9)
    h2, Wr2 = workloads.radial_inputs(wl2.E, K, L, C, seed=6)
    p2 = DeviceProblem(wl2, need=("G",))
    gx2, gh2, gr2 = (np_(t) for t in run_vjp(p2, h2, Wr2))
    r2 = oracle.vjp_radial(L, wl2.row_ptr, wl2.src, wl2.vec, wl2.x, h2, Wr2, wl2.G)
    for got, ref in zip((gx2, gh2, gr2), r2[:3]):
        assert rel_err(got, ref) < FP32_TOL


def test_radial_vjp_bf16_features():
    say("vjp-bf16")
    L, C, K = 3, 128, 8
    wl = workloads.small(L, C, 19, 12, seed=41)
    h, Wr = workloads.radial_inputs(wl.E, K, L, C, seed=7)
    p = DeviceProblem(wl, bf16=True, need=("G",))
    gx, gh, gr = (np_(t) for t in run_vjp(p, h, Wr))
    ref = oracle.vjp_radial(L, wl.row_ptr, wl.src, wl.vec, p.x_seen, h, Wr, wl.G)
    for name, got, r in zip(("gx", "gh", "gr"), (gx, gh, gr), ref[:3]):
        assert rel_err(got, r) < FP32_TOL, (name, rel_err(got, r))


def test_radial_vjp_argument_checks():
    import torch
    say("vjp-args")
    wl = workloads.small(1, 8, 6, 3, seed=2)
    p = DeviceProblem(wl, need=("G",))
    gr = p.empty(wl.E, 3)
    for K in (0, 9):
        h = torch.zeros(wl.E, max(K, 1), device="cuda")
        Wr = torch.zeros(max(K, 1), p.plan.P, wl.C, device="cuda")
        with pytest.raises(p.etp.EtpError) as ei:
            p.etp.etp_edge_conv_vjp_radial(p.plan, p.graph, p.vec, p.x, h if K else None, Wr if K else None, p.G,
                                           grad_vec=gr)
        assert ei.value.status in (p.etp.ETP_ERR_UNSUPPORTED, p.etp.ETP_ERR_INVALID_ARGUMENT)


def test_radial_vjp_micro_full_size_sampled():
    """The microbenchmark's VJP with 8 basis functions at full size; source
    nodes sampled, their out-edges recomputed by the oracle."""
    say("vjp-micro")
    wl = workloads.get("micro")
    K = 8
    h, Wr = workloads.radial_inputs(wl.E, K, wl.L, wl.C, seed=11)
    p = DeviceProblem(wl, need=("G",))
    gx, gh, gr = (np_(t) for t in run_vjp(p, h, Wr))
    g = np.random.default_rng(4)
    cols = np.unique(np.concatenate([[0, wl.n - 1], g.choice(wl.n, 6, replace=False)]))
    rp2, eidx2 = src_subgraph(wl, cols)
    rgx, rgh, rgr, _ = oracle.vjp_radial(wl.L, rp2, wl.src[eidx2], wl.vec[eidx2], wl.x, h[eidx2], Wr, wl.G)
    assert rel_err(gx[cols], rgx[cols]) < FP32_TOL
    assert rel_err(gh[eidx2], rgh) < FP32_TOL
    assert rel_err(gr[eidx2], rgr) < FP32_TOL
