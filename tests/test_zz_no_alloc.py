"""The transpose entry point that allocates nothing
(etp_csr_transpose_noalloc, workspace in a fixed device array inside the
library) against etp_csr_transpose with a caller workspace: bit for bit,
through the C ABI, on consecutive calls whose second input is smaller (the
array keeps the first call's contents), and against the oracle's stable
transpose."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_common import dev

pytestmark = pytest.mark.gpu


def _both(wl):
    import torch
    from equivariant_interatomic_potentials_amd import etp
    E, n = wl.E, wl.n
    row_ptr, src = dev(wl.row_ptr.astype(np.int32)), dev(wl.src.astype(np.int32))
    g = etp.Graph(wl.n_dst, n, row_ptr, src)
    out = []
    for noalloc in (False, True):
        sp = torch.full((n + 1,), -7, dtype=torch.int32, device="cuda")
        pm = torch.full((max(E, 1),), -7, dtype=torch.int32, device="cuda")
        pd = torch.full((max(E, 1),), -7, dtype=torch.int32, device="cuda")
        if noalloc:
            etp.etp_csr_transpose_noalloc(g, sp, pm[:E], pd[:E])
        else:
            ws = torch.empty(etp.etp_csr_transpose_workspace(n) // 4 + 1, dtype=torch.int32, device="cuda")
            etp.etp_csr_transpose(g, sp, pm[:E], pd[:E], ws)
        torch.cuda.synchronize()
        out.append(tuple(t.cpu().numpy() for t in (sp, pm[:E], pd[:E])))
    return out


def test_noalloc_transpose_matches_workspace_call():
    cases = [workloads.get("micro"),                          # 1024 sources, 131072 edges
             workloads.small(2, 8, 37, 9, seed=3),             # ragged, empty rows
             workloads.bipartite(1, 8, 3, 300, 150, 300, seed=1),  # few destinations, long destination rows
             workloads.bipartite(1, 8, 5000, 3, 2, 3, seed=4),     # source rows above the LDS sort tile
             workloads.small(1, 8, 5, 0, seed=2)]              # no edges
    for wl in cases:
        print("noalloc transpose", wl.name, wl.n_dst, wl.n, wl.E, flush=True)
        (rs, rp, rd), (ns, np_, nd) = _both(wl)
        assert np.array_equal(rs, ns) and np.array_equal(rp, np_) and np.array_equal(rd, nd)
        sp, pm, pd = oracle.transpose(wl.row_ptr, wl.src, wl.n)
        assert np.array_equal(ns, sp) and np.array_equal(np_, pm) and np.array_equal(nd, pd)


def test_noalloc_transpose_on_a_stream():
    """The same call on a non-default stream (default priority) gives the same result."""
    import torch
    from equivariant_interatomic_potentials_amd import etp
    wl = workloads.small(3, 16, 200, 40, seed=9)
    E, n = wl.E, wl.n
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        row_ptr, src = dev(wl.row_ptr.astype(np.int32)), dev(wl.src.astype(np.int32))
        sp = torch.empty(n + 1, dtype=torch.int32, device="cuda")
        pm = torch.empty(E, dtype=torch.int32, device="cuda")
        pd = torch.empty(E, dtype=torch.int32, device="cuda")
        etp.etp_csr_transpose_noalloc(etp.Graph(wl.n_dst, n, row_ptr, src), sp, pm, pd, stream=s)
    s.synchronize()
    ref = oracle.transpose(wl.row_ptr, wl.src, wl.n)
    for got, want in zip((sp, pm, pd), ref):
        assert np.array_equal(got.cpu().numpy(), want)
