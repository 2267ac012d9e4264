"""Benchmark of the fused edge tensor-product convolution on one MI355X.

Headline workload: the 32768-atom diamond solid (16^3 conventional cells,
a = 3.567 A, Gaussian jitter 0.05 A, periodic, 6.0 A cutoff: about 158
neighbours per atom and 5.17 M edges; C = 128 channels, l_max = 3) -- the
diamond system of "How does FlashCart make equivariant interatomic potentials
faster and more accurate?" (SPICE-MACE-OFF section), the largest
configuration that fits one GPU. The node features are fp32 for the value
(a second run stores them in bf16, fp32 arithmetic either way).

One step = one pass of the whole device path over that graph:

    CSR transpose -> forward -> VJP (gx, gw, forces) -> VJP-of-VJP (dx, dw, dr, dG)

value = edges per second of forward + VJP, E / (t_fwd + t_vjp), with every
input resident in HBM; the per-op times come from HIP events recorded on the
launch stream around each call inside the timed region. Every op is also
reported against its compulsory bytes (each tensor touched once) and
algorithmic FLOPs; the roofline object is the op that takes the most time.
The other workloads (tiny, micro, micro3, micro4, water) are timed the same
way under "configs". The float64 oracle is timed on the host on a bounded
sample of destination rows of the diamond graph.

Per-edge arrays too large for the device budget (the VJP-of-VJP cotangent
on w, 90 GB in fp32 at the diamond) are drawn per destination-row chunk on
the GPU outside the timed ops; each chunk runs on its own sub-CSR and
transpose, node gradients accumulating across chunks.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload diamond]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "edges/sec for fused edge TP conv (fwd, fwd+VJP) + % of HBM/VALU roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
VALU_PEAK_TFLOPS = 157.3       # MI355X fp32 vector (packed); 78.6 without packing
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix-core peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
WORKLOADS = {
    "diamond": "32768-atom diamond (16^3 cells, a=3.567 A, jitter 0.05 A), 6 A cutoff, C=128, l_max=3",
    "micro": "1024 nodes x 128 random neighbours (131072 edges), C=128, l_max=2",
    "micro3": "1024 nodes x 128 random neighbours (131072 edges), C=128, l_max=3",
    "micro4": "1024 nodes x 128 random neighbours (131072 edges), C=128, l_max=4",
    "water": "5184-atom water box, 6 A cutoff, C=64, l_max=2",
    "tiny": "32 nodes x 8 random neighbours (256 edges), C=8, l_max=1",
}
CONFIG_ORDER = ("tiny", "micro", "micro3", "micro4", "water", "diamond")
OPS = ("transpose", "fwd", "vjp", "vjp2")


def table_counts(L):
    """(P, nnz, pairs, Din, Dout, per-path 2l1+1 and 2l3+1) from the library's own tables."""
    from equivariant_interatomic_potentials_amd import etp
    plan = etp.etp_plan_create(L, 8)
    t = etp.etp_plan_tables(plan)
    P = plan.P
    pairs = 0
    d1 = []
    d3 = []
    for p in range(P):
        l1, l2, l3 = t["paths"][p]
        ms = t["cg_m"][t["cg_ptr"][p]:t["cg_ptr"][p + 1]]
        pairs += len({(int(a), int(c)) for a, _, c in ms})
        d1.append(2 * l1 + 1)
        d3.append(2 * l3 + 1)
    return dict(P=P, nnz=plan.nnz, pairs=pairs, Din=plan.din_rows, Dout=plan.dout_rows,
                d1=np.array(d1), d3=np.array(d3))


def compulsory(L, C, N, E, n_src, xb=4):
    """Per-op compulsory HBM bytes (every tensor the op must read or write,
    touched once; x in xb bytes per value) and algorithmic FLOPs (2 per FMA of
    the sparse contraction, per edge and channel: fwd nnz + sum_p min(2l1+1,
    2l3+1); VJP 2 nnz + pairs + 3 sum_p (2l1+1); VJP-of-VJP 6 nnz + 2 pairs +
    9 sum_p (2l1+1)). The VJP-of-VJP is one op: its destination and source
    halves together must touch w, W' and dw once each."""
    k = table_counts(L)
    P, nnz, pairs, Din, Dout = k["P"], k["nnz"], k["pairs"], k["Din"], k["Dout"]
    w = 4.0 * E * P * C
    xin = float(n_src) * Din * C * xb
    x32 = 4.0 * n_src * Din * C
    out = 4.0 * N * Dout * C
    vec = 12.0 * E
    idx = 4.0 * E
    offs = 4.0 * (N + 1)
    toffs = 4.0 * (n_src + 1)
    by = {
        "transpose": 4 * idx + toffs + offs,
        "fwd": w + xin + out + vec + idx + offs,
        "vjp": 2 * w + xin + x32 + out + 2 * vec + 2 * idx + offs + toffs,
        "vjp2": 3 * w + xin + 2 * x32 + 2 * out + 3 * vec + 3 * idx + offs + toffs,
    }
    sum_min = int(np.minimum(k["d1"], k["d3"]).sum())
    s1 = int(k["d1"].sum())
    fma_ch = {"transpose": 0, "fwd": nnz + sum_min, "vjp": 2 * nnz + pairs + 3 * s1,
              "vjp2": 6 * nnz + 2 * pairs + 9 * s1}
    fl = {op: 2.0 * fma_ch[op] * C * E for op in by}
    return by, fl


def roof(byts, flops, t):
    """Roofline of one op: the larger of its HBM and VALU times at peak over
    the measured time."""
    th = byts / (HBM_PEAK_GBS * 1e9)
    tv = flops / (VALU_PEAK_TFLOPS * 1e12)
    if th >= tv:
        return {"bound": "hbm", "achieved": round(byts / t / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(th / t, 4)}
    return {"bound": "alu", "achieved": round(flops / t / 1e12, 2), "peak": VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tv / t, 4)}


# the device code of the timed step (transpose, forward, VJP, VJP-of-VJP)
# and the headers it includes; the host-side C-ABI file and the kernels of
# the calls around the convolution are left out (they do not change what the
# step's kernels move)
STEP_SOURCES = ("etp_graph.hip", "etp_dst.hip", "etp_src.hip", "etp_bwd.hip", "etp_device.hpp",
                "etp_conv_common.hpp", "etp_groups.hpp", "etp_tables.hpp")


def kernel_source_hash():
    """Hash of the step's device-code sources."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "equivariant_interatomic_potentials_amd", "csrc")
    for f in STEP_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, op):
    """HBM bytes per call of `op` on `workload` from committed rocprofv3
    counter runs, if they were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_call", {}).get(workload, {}).get(op)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ------------------------------------------------------------ the step

class Problem:
    """One workload resident on the GPU: graph, transpose, features, weights,
    cotangents and outputs, with the step's ops as closures. Per-edge
    cotangents that do not fit beside w, gw and dw are drawn per chunk of
    destination rows (outside the timed ops)."""

    def __init__(self, name, bf16=False, shared=None, bwd="auto"):
        import torch

        import workloads
        from equivariant_interatomic_potentials_amd import etp
        self.etp, self.torch = etp, torch
        self.name = name
        self.bf16 = bf16
        # the backward: "auto" = the workspace entry points with the library's
        # choice of formulation per shape; "dst" forces the walk over each
        # destination's in-edges (node gradient through a per-edge workspace);
        # "src" = the entry points without workspace (each source's out-edges)
        self.bwd = bwd
        wl = shared["wl"] if shared else workloads.get(name)
        self.wl = wl
        L, C, N, E, n_src, P = wl.L, wl.C, wl.n_dst, wl.E, wl.n, wl.P
        self.L, self.C, self.N, self.E, self.n_src, self.P = L, C, N, E, n_src, P
        self.plan = etp.etp_plan_create(L, C, etp.ETP_BF16 if bf16 else etp.ETP_F32)
        cuda = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        if shared:
            for k in ("row_ptr", "src", "vec", "ggv", "w", "G", "ggx", "x32", "src_ptr", "perm", "perm_dst", "tws",
                      "chunks", "out", "gx", "gr", "dx", "dr", "dG", "gw", "ggw_full", "ggw_buf", "bws"):
                setattr(self, k, shared[k])
        else:
            self.row_ptr, self.src, self.vec = cuda(wl.row_ptr), cuda(wl.src), cuda(wl.vec)
            self.ggv = cuda(wl.ggvec)
            # per-edge weights drawn on the device (the diamond's are 90 GB)
            self.w = workloads.device_normal((E, P, C), wl.seed, "w", 0, 1.0 / np.sqrt(P))
            self.G = workloads.device_normal((N, wl.Dout, C), wl.seed, "G", 0)
            self.ggx = workloads.device_normal((n_src, wl.Din, C), wl.seed, "ggx", 0)
            self.x32 = cuda(wl.x)
            self.src_ptr = torch.empty(n_src + 1, dtype=torch.int32, device="cuda")
            self.perm = torch.empty(E, dtype=torch.int32, device="cuda")
            self.perm_dst = torch.empty(E, dtype=torch.int32, device="cuda")
            self.tws = torch.empty(etp.etp_csr_transpose_workspace(n_src) // 4 + 1, dtype=torch.int32,
                                   device="cuda")
            self.out = torch.empty(N, wl.Dout, C, device="cuda")
            self.gx = torch.empty(n_src, wl.Din, C, device="cuda")
            self.gr = torch.empty(E, 3, device="cuda")
            self.dx, self.dr, self.dG = torch.empty_like(self.gx), torch.empty_like(self.gr), torch.empty_like(self.out)
            # gw (VJP output) and dw (VJP-of-VJP output) share one buffer: a
            # step writes gw, then dw over it
            self.gw = torch.empty(E, P, C, device="cuda")
            # the destination-side backward's workspace (one Din-row block per
            # edge and the bond-vector partials of its path groups), allocated
            # for both formulations so that either can run
            g_sz = etp.Graph(N, n_src, self.row_ptr, self.src)
            self.bws = torch.empty(etp.etp_workspace_size(self.plan, etp.ETP_OP_VJP_WS, g_sz) // 4, device="cuda")
            self._plan_chunks()
        self.x = self.x32.to(torch.bfloat16) if bf16 else self.x32
        self.g0 = etp.Graph(N, n_src, self.row_ptr, self.src)
        self.g = etp.Graph(N, n_src, self.row_ptr, self.src, self.src_ptr, self.perm, self.perm_dst)

    def shared(self):
        return {k: getattr(self, k) for k in (
            "wl", "row_ptr", "src", "vec", "ggv", "w", "G", "ggx", "x32", "src_ptr", "perm", "perm_dst", "tws",
            "chunks", "out", "gx", "gr", "dx", "dr", "dG", "gw", "ggw_full", "ggw_buf", "bws")}

    def _plan_chunks(self):
        """Destination-row chunks for the VJP-of-VJP: one when its per-edge
        cotangent fits beside everything else, else the fewest that fit."""
        import torch

        import workloads
        etp, wl = self.etp, self.wl
        free, _ = torch.cuda.mem_get_info()
        per_edge = 4.0 * self.P * self.C
        margin = 6e9
        n = 1
        while n < 64 and per_edge * self.E / n > free - margin:
            n *= 2
        self.n_chunks = n
        bounds = np.linspace(0, self.N, n + 1).astype(int)
        self.chunks = []
        for c in range(n):
            r0, r1 = int(bounds[c]), int(bounds[c + 1])
            e0, e1 = int(wl.row_ptr[r0]), int(wl.row_ptr[r1])
            ch = {"r0": r0, "r1": r1, "e0": e0, "e1": e1}
            if n > 1:
                rp = torch.from_numpy((wl.row_ptr[r0:r1 + 1] - e0).astype(np.int32)).cuda()
                src = self.src[e0:e1]
                sp = torch.empty(self.n_src + 1, dtype=torch.int32, device="cuda")
                pm = torch.empty(e1 - e0, dtype=torch.int32, device="cuda")
                pd = torch.empty(e1 - e0, dtype=torch.int32, device="cuda")
                etp.etp_csr_transpose(etp.Graph(r1 - r0, self.n_src, rp, src), sp, pm, pd, self.tws)
                ch["g"] = etp.Graph(r1 - r0, self.n_src, rp, src, sp, pm, pd)
            self.chunks.append(ch)
        if n == 1:
            self.ggw_full = workloads.device_normal((self.E, self.P, self.C), wl.seed, "ggw", 0)
            self.ggw_buf = None
        else:
            self.ggw_full = None
            emax = max(ch["e1"] - ch["e0"] for ch in self.chunks)
            self.ggw_buf = torch.empty(emax * self.P * self.C, device="cuda")
        torch.cuda.synchronize()

    def fill_ggw(self, c):
        """The chunk's cotangent on w, drawn in place on the device."""
        import workloads
        ch = self.chunks[c]
        n = (ch["e1"] - ch["e0"]) * self.P * self.C
        buf = self.ggw_buf[:n].view(ch["e1"] - ch["e0"], self.P, self.C)
        workloads.device_normal_(buf, self.wl.seed, "ggw", c)
        return buf

    def step(self, ev=None, ops=OPS):
        """One pass of the path; ev[op] is a list of (start, end) event pairs
        that receive the op's calls."""
        etp = self.etp
        plan, g = self.plan, self.g

        def timed(op, f):
            if ev is None:
                f()
                return
            a, b = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            ev[op].append((a, b))

        if "transpose" in ops:
            timed("transpose", lambda: etp.etp_csr_transpose(self.g0, self.src_ptr, self.perm, self.perm_dst,
                                                             self.tws))
        if "fwd" in ops:
            timed("fwd", lambda: etp.etp_edge_conv_fwd(plan, g, self.vec, self.x, self.w, self.out))
        dst = self.bwd != "src"
        force = etp.ETP_FLAG_DST_PASS if self.bwd == "dst" else 0
        if "vjp" in ops:
            if dst:
                timed("vjp", lambda: etp.etp_edge_conv_vjp_ws(plan, g, self.vec, self.x, self.w, self.G, self.gx,
                                                              self.gw, self.gr, self.bws, force))
            else:
                timed("vjp", lambda: etp.etp_edge_conv_vjp(plan, g, self.vec, self.x, self.w, self.G, self.gx,
                                                           self.gw, self.gr))
        if "vjp2" in ops:
            def vjp2(gr_, vec, w, G, ggw, ggv, dw, dr, dG, acc):
                if dst:
                    etp.etp_edge_conv_vjp2_ws(plan, gr_, vec, self.x, w, G, self.ggx, ggw, ggv, self.dx, dw, dr, dG,
                                              self.bws, acc | force)
                else:
                    etp.etp_edge_conv_vjp2(plan, gr_, vec, self.x, w, G, self.ggx, ggw, ggv, self.dx, dw, dr, dG,
                                           acc)
            if len(self.chunks) == 1:
                timed("vjp2", lambda: vjp2(g, self.vec, self.w, self.G, self.ggw_full, self.ggv, self.gw, self.dr,
                                           self.dG, 0))
            else:
                for c, ch in enumerate(self.chunks):
                    ggw = self.fill_ggw(c)
                    r0, r1, e0, e1 = ch["r0"], ch["r1"], ch["e0"], ch["e1"]
                    acc = etp.ETP_FLAG_ACCUMULATE if c else 0
                    timed("vjp2", lambda: vjp2(ch["g"], self.vec[e0:e1], self.w[e0:e1], self.G[r0:r1], ggw,
                                               self.ggv[e0:e1], self.gw[e0:e1], self.dr[e0:e1], self.dG[r0:r1], acc))

    def run(self, steps, warmup, ops=OPS):
        """warmup untimed steps, then `steps` timed ones; per-op mean ms over
        the steps (an op's chunks summed) and wall ms per step."""
        torch = self.torch
        for _ in range(warmup):
            self.step(None, ops)
        torch.cuda.synchronize()
        evs = []
        t0 = time.perf_counter()
        for _ in range(steps):
            ev = {op: [] for op in ops}
            self.step(ev, ops)
            evs.append(ev)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per_op = {op: float(np.mean([sum(a.elapsed_time(b) for a, b in ev[op]) for ev in evs])) for op in ops}
        return per_op, wall / steps * 1e3

    def report(self, per_op):
        """Per-op ms, edges/s and roofline fraction against compulsory bytes."""
        xb = 2 if self.bf16 else 4
        by, fl = compulsory(self.L, self.C, self.N, self.E, self.n_src, xb)
        rep = {}
        for op, ms in per_op.items():
            t = ms * 1e-3
            r = {"ms": round(ms, 4), "edges_per_s": self.E / t, "algo_GBps": round(by[op] / t / 1e9, 1),
                 "algo_TFLOPs": round(fl[op] / t / 1e12, 2)}
            if op != "transpose":
                rf = roof(by[op], fl[op], t)
                r.update({"bound": rf["bound"], "frac": rf["frac"],
                          "compulsory_B_per_edge": round(by[op] / self.E, 1),
                          "flop_per_edge": round(fl[op] / self.E, 1)})
            rep[op] = r
        return rep, by, fl


def other_bwd(p, steps, warmup):
    """The VJP and VJP-of-VJP in each forced formulation (destination side,
    source side), on the same buffers: ms, edges/s and roofline fraction."""
    out = {}
    for b in ("dst", "src"):
        alt = Problem(p.name, bf16=p.bf16, shared=p.shared(), bwd=b)
        per, _ = alt.run(steps, warmup, ops=("vjp", "vjp2"))
        rep, _, _ = alt.report(per)
        out[b] = {op: {k: rep[op][k] for k in ("ms", "edges_per_s", "bound", "frac")} for op in rep}
    return out


def config_entry(name, steps, warmup, bwd):
    """A non-headline workload: fwd, fwd+VJP and per-op figures (and the
    other backward formulation beside them)."""
    import torch
    p = Problem(name, bwd=bwd)
    per_op, ms_step = p.run(steps, warmup)
    rep, _, _ = p.report(per_op)
    fwd_vjp = p.E / ((per_op["fwd"] + per_op["vjp"]) * 1e-3)
    d = {"workload": WORKLOADS[name], "n_nodes": p.N, "n_edges": p.E, "channels": p.C, "l_max": p.L,
         "ms_per_step": round(ms_step, 4), "fwd_edges_per_s": rep["fwd"]["edges_per_s"],
         "fwd_vjp_edges_per_s": fwd_vjp, "vjp2_chunks": len(p.chunks), "bwd": p.bwd, "ops": rep,
         "other_bwd": other_bwd(p, steps, warmup)}
    del p
    torch.cuda.empty_cache()
    return d


# ------------------------------------------------- calls beside the step

def time_calls(f, reps, warm=2):
    import torch
    for _ in range(warm):
        f()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        f()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e-3


def time_radial(etp, p, reps, K=8):
    """The forward and VJP with radial weights formed in the kernel (w = h Wr,
    K basis functions) on the same graph and features as the step: ms per
    call against the plain calls that read w (and write gw), each timed the
    same way (back-to-back calls) just before the radial one. Algorithmic
    bytes: the plain call's with the E P C weight streams replaced by h (and
    grad_h) and Wr; FLOPs: the plain call's plus 2 K per (edge, path,
    channel) to form w (and 2 K more for grad_h)."""
    import torch

    import workloads
    L, C, E, P = p.L, p.C, p.E, p.P
    h, Wr = workloads.radial_inputs(E, K, L, C, seed=0)
    h, Wr = torch.from_numpy(h).cuda(), torch.from_numpy(Wr).cuda()
    y = torch.empty_like(p.out)
    t_plain = time_calls(lambda: etp.etp_edge_conv_fwd(p.plan, p.g, p.vec, p.x, p.w, y), reps, 3)
    t = time_calls(lambda: etp.etp_edge_conv_fwd_radial(p.plan, p.g, p.vec, p.x, h, Wr, y), reps, 3)
    by, fl = compulsory(L, C, p.N, E, p.n_src)
    byts = by["fwd"] - 4.0 * E * P * C + 4.0 * (E * K + K * P * C)
    flops = fl["fwd"] + 2.0 * K * P * C * E
    res = {"ms": round(t * 1e3, 4), "edges_per_s": E / t, "n_basis": K,
           "plain_fwd_ms": round(t_plain * 1e3, 4), "speedup_vs_fwd": round(t_plain / t, 3),
           "algo_GBps": byts / t / 1e9,
           "algo_TFLOPs": flops / t / 1e12, "hbm_frac": byts / t / 1e9 / HBM_PEAK_GBS,
           "valu_frac": flops / t / 1e12 / VALU_PEAK_TFLOPS}
    gx, gh, gr = torch.empty_like(p.gx), torch.empty(E, K, device="cuda"), torch.empty_like(p.gr)
    tv_plain = time_calls(lambda: etp.etp_edge_conv_vjp_ws(p.plan, p.g, p.vec, p.x, p.w, p.G, gx, p.gw, gr, p.bws),
                          reps)
    tv = time_calls(lambda: etp.etp_edge_conv_vjp_radial(p.plan, p.g, p.vec, p.x, h, Wr, p.G, gx, gh, gr), reps)
    vb = by["vjp"] - 8.0 * E * P * C + 4.0 * (2 * E * K + K * P * C)
    vf = fl["vjp"] + 4.0 * K * P * C * E
    res.update({"vjp_ms": round(tv * 1e3, 4), "plain_vjp_ms": round(tv_plain * 1e3, 4),
                "vjp_speedup_vs_vjp": round(tv_plain / tv, 3),
                "vjp_hbm_frac": vb / tv / 1e9 / HBM_PEAK_GBS, "vjp_valu_frac": vf / tv / 1e12 / VALU_PEAK_TFLOPS})
    # the VJP with the weight gradient (grad_Wr), and the VJP-of-VJP with and
    # without d_Wr (cotangents on grad_x, grad_h, grad_vec)
    wsz = etp.etp_workspace_size(p.plan, etp.ETP_OP_RADIAL_WGRAD, p.g)
    ws = torch.empty(wsz, dtype=torch.uint8, device="cuda")
    gWr = torch.empty_like(Wr)
    tw = time_calls(lambda: etp.etp_edge_conv_vjp_radial_wgrad(p.plan, p.g, p.vec, p.x, h, Wr, p.G, gx, gh, gr, gWr,
                                                               ws), reps)
    Hp = torch.randn_like(h)
    dx, dh, dr, dG = torch.empty_like(gx), torch.empty_like(gh), torch.empty_like(gr), torch.empty_like(p.out)
    t2 = time_calls(lambda: etp.etp_edge_conv_vjp2_radial(p.plan, p.g, p.vec, p.x, h, Wr, p.G, p.ggx, Hp, p.ggv,
                                                          dx, dh, dr, dG), reps)
    t2w = time_calls(lambda: etp.etp_edge_conv_vjp2_radial_wgrad(p.plan, p.g, p.vec, p.x, h, Wr, p.G, p.ggx, Hp,
                                                                 p.ggv, dx, dh, dr, dG, gWr, ws), reps)
    # VJP-of-VJP bytes: the plain op's with the three E P C streams replaced by
    # h, H', dh and Wr; FLOPs: the plain op's plus 2 K per (edge, path,
    # channel) for each of w and W' (and dh)
    b2 = by["vjp2"] - 12.0 * E * P * C + 4.0 * (3 * E * K + K * P * C)
    f2 = fl["vjp2"] + 6.0 * K * P * C * E
    res.update({"vjp_wgrad_ms": round(tw * 1e3, 4), "vjp2_ms": round(t2 * 1e3, 4),
                "vjp2_wgrad_ms": round(t2w * 1e3, 4), "vjp2_hbm_frac": b2 / t2 / 1e9 / HBM_PEAK_GBS,
                "vjp2_valu_frac": f2 / t2 / 1e12 / VALU_PEAK_TFLOPS})
    del ws
    return res


def time_channel_mix(etp, plan, out, L, C, N, reps):
    """The per-irrep channel mixing after the convolution (outside the step):
    ms per call, algorithmic bytes (conv output, W, result, each once) and
    FLOPs (2 per multiply-add of the per-order products)."""
    import torch
    rows = etp.mix_rows(plan)
    g = torch.Generator(device="cuda")
    g.manual_seed(12345)
    W = torch.randn(sum(rows) * C * C, generator=g, device="cuda") / float(np.sqrt(C))
    y = torch.empty(N, (L + 1) ** 2, C, device="cuda")
    t = time_calls(lambda: etp.etp_channel_mix(plan, out, W, y), reps, 3)
    byts = 4.0 * (out.numel() + W.numel() + y.numel())
    flops = 2.0 * sum(N * (2 * l + 1) * rows[l] * C * C for l in range(L + 1))
    res = {"ms": round(t * 1e3, 4), "algo_GBps": byts / t / 1e9, "algo_TFLOPs": flops / t / 1e12,
           "hbm_frac": byts / t / 1e9 / HBM_PEAK_GBS, "mfma_frac": flops / t / 1e12 / MFMA_F32_PEAK_TFLOPS,
           "bound": "mfma" if flops / (MFMA_F32_PEAK_TFLOPS * 1e12) > byts / (HBM_PEAK_GBS * 1e9) else "hbm"}
    gin = torch.empty_like(out)
    tv = time_calls(lambda: etp.etp_channel_mix_vjp(plan, y, W, gin), reps)
    res.update({"vjp_ms": round(tv * 1e3, 4), "vjp_mfma_frac": flops / tv / 1e12 / MFMA_F32_PEAK_TFLOPS})
    # bf16 weights (W read at 2 bytes; its own dtype's peak)
    Wb = W.to(torch.bfloat16)
    tb = time_calls(lambda: etp.etp_channel_mix_ex(plan, out, Wb, y), reps, 3)
    tbv = time_calls(lambda: etp.etp_channel_mix_vjp_ex(plan, y, Wb, gin), reps, 3)
    bb = byts - 2.0 * W.numel()
    res["bf16"] = {"ms": round(tb * 1e3, 4), "vjp_ms": round(tbv * 1e3, 4), "hbm_frac": bb / tb / 1e9 / HBM_PEAK_GBS,
                   "mfma_frac": flops / tb / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                   "vjp_hbm_frac": bb / tbv / 1e9 / HBM_PEAK_GBS}
    # the weight gradient (a sum over the nodes: the same FLOPs; reads the
    # input and the cotangent once, writes grad_W)
    wws = etp.mix_wgrad_workspace(plan, N)
    gW = torch.empty_like(W)
    tg = time_calls(lambda: etp.etp_channel_mix_wgrad(plan, out, y, gW, wws), reps, 3)
    res.update({"wgrad_ms": round(tg * 1e3, 4), "wgrad_mfma_frac": flops / tg / 1e12 / MFMA_F32_PEAK_TFLOPS})
    return res


def time_edge_forces(etp, g, gr, N, n_src, E, reps):
    """Edge-to-atom force assembly from the VJP's grad_vec (outside the step):
    ms per call; algorithmic bytes = grad_vec, perm, both offset arrays and the
    forces, each once."""
    import torch
    n = max(N, n_src)
    F = torch.empty(n, 3, device="cuda")
    t = time_calls(lambda: etp.etp_edge_forces(g, gr, F), reps, 3)
    byts = 12.0 * E + 4.0 * E + 4.0 * (N + 1) + 4.0 * (n_src + 1) + 12.0 * n
    return {"ms": round(t * 1e3, 4), "algo_GBps": byts / t / 1e9, "hbm_frac": byts / t / 1e9 / HBM_PEAK_GBS,
            "bound": "hbm"}


def time_neighbor_list(etp, pos_np, box, rc, reps):
    """Periodic neighbour list (outside the step): ms of the count call and of
    the fill call; algorithmic bytes = positions in, row_ptr out (count) and
    positions + row_ptr in, src + vec out (fill)."""
    import torch
    n = pos_np.shape[0]
    pos = torch.from_numpy(np.ascontiguousarray(pos_np, np.float32)).cuda()
    ws = torch.empty(etp.etp_neighbor_workspace(n, box, rc), dtype=torch.uint8, device="cuda")
    rp = torch.empty(n + 1, dtype=torch.int32, device="cuda")
    etp.etp_neighbor_count(pos, box, rc, rp, ws)
    E = int(rp[n].item())
    src = torch.empty(E, dtype=torch.int32, device="cuda")
    vec = torch.empty(E, 3, device="cuda")
    for _ in range(3):
        etp.etp_neighbor_count(pos, box, rc, rp, ws)
        etp.etp_neighbor_fill(pos, box, rc, rp, E, src, vec, ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tc = tf = 0.0
    for _ in range(reps):
        ev[0].record()
        etp.etp_neighbor_count(pos, box, rc, rp, ws)
        ev[1].record()
        etp.etp_neighbor_fill(pos, box, rc, rp, E, src, vec, ws)
        ev[2].record()
        torch.cuda.synchronize()
        tc += ev[0].elapsed_time(ev[1])
        tf += ev[1].elapsed_time(ev[2])
    tc, tf = tc / reps * 1e-3, tf / reps * 1e-3
    bc = 12.0 * n + 4.0 * (n + 1)
    bf = 12.0 * n + 4.0 * (n + 1) + 16.0 * E
    return {"atoms": n, "edges": E, "cutoff": rc, "count_ms": round(tc * 1e3, 4), "fill_ms": round(tf * 1e3, 4),
            "edges_per_s": E / (tc + tf), "fill_algo_GBps": bf / tf / 1e9,
            "algo_GBps": (bc + bf) / (tc + tf) / 1e9, "hbm_frac": (bc + bf) / (tc + tf) / 1e9 / HBM_PEAK_GBS,
            "bound": "alu"}


def time_edge_tp(etp, plan, L, C, E, Din, P, Dout, vec, w, reps):
    """Edge-local tensor product on the step's edges (outside the step): ms of
    the forward, the VJP (gV, gw, gr) and the VJP-of-VJP; algorithmic bytes =
    every input and output once."""
    import torch

    import workloads
    V = workloads.device_normal((E, Din, C), 3, "x", 8192)
    G = workloads.device_normal((E, Dout, C), 4, "G", 8192)
    out = torch.empty(E, Dout, C, device="cuda")
    gV, gw, gr = torch.empty_like(V), torch.empty_like(w), torch.empty(E, 3, device="cuda")
    ggV, ggw, ggv = torch.randn_like(V), torch.randn_like(w), torch.randn(E, 3, device="cuda")
    dG = torch.empty_like(G)
    res = {}
    for name, f, byts in (
            ("fwd", lambda: etp.etp_edge_tp_fwd(plan, vec, V, w, out), 4.0 * E * (3 + Din * C + P * C + Dout * C)),
            ("vjp", lambda: etp.etp_edge_tp_vjp(plan, vec, V, w, G, gV, gw, gr),
             4.0 * E * (6 + 2 * Din * C + 2 * P * C + Dout * C)),
            ("vjp2", lambda: etp.etp_edge_tp_vjp2(plan, vec, V, w, G, ggV, ggw, ggv, gV, gw, gr, dG),
             4.0 * E * (3 + 2 * Din * C + 2 * P * C + Dout * C + 3 + Din * C + P * C + 3 + Dout * C))):
        t = time_calls(f, reps)
        res[name + "_ms"] = round(t * 1e3, 4)
        res[name + "_algo_GBps"] = byts / t / 1e9
        res[name + "_hbm_frac"] = byts / t / 1e9 / HBM_PEAK_GBS
    res.update({"edges": E, "l_max": L, "channels": C, "bound": "hbm"})
    del V, G, out, gV, gw, gr, ggV, ggw, ggv, dG
    torch.cuda.empty_cache()
    return res


def time_node_product(etp, L, nu, reps, n=4096, C=128):
    """Node-local correlation product (outside the step) at the FlashCart
    page's node-local benchmark size: ms per call and VALU FLOPs per call =
    n C (nu - 1) (n_prod + 2 nnz + 2 Dout + D): one product B[l1, m1] A[l2, m2]
    per distinct (l1, m1, l2, m2) of the CG table (shared by the paths that
    differ only in l3), one FMA per CG entry, one FMA per output row of a path
    for its weight, one add per row of the running sum."""
    import torch

    import workloads
    plan = etp.etp_plan_create(L, C)
    tb = etp.etp_plan_tables(plan)
    prods = set()
    for p, (l1, l2, _) in enumerate(tb["paths"]):
        for m1, m2, _ in tb["cg_m"][tb["cg_ptr"][p]:tb["cg_ptr"][p + 1]]:
            prods.add((int(l1), int(m1), int(l2), int(m2)))
    nnz, dout, D = len(tb["cg_val"]), int(tb["out_off"][-1]), (L + 1) ** 2
    A_np, W_np = workloads.node_features(n, L, C, nu, seed=0)
    A = torch.from_numpy(A_np).cuda()
    W = torch.from_numpy(W_np).cuda()
    out = torch.empty_like(A)
    t = time_calls(lambda: etp.etp_node_product(plan, A, W, out, nu), reps, 3)
    f_step = len(prods) + 2 * nnz + 2 * dout + D
    flops = float(n) * C * (nu - 1) * f_step
    byts = 4.0 * (2 * n * D * C + (nu - 1) * len(tb["paths"]) * C)
    res = {"nodes": n, "channels": C, "l_max": L, "corr_order": nu, "ms": round(t * 1e3, 4),
           "algo_TFLOPs": flops / t / 1e12, "valu_frac": flops / t / 1e12 / VALU_PEAK_TFLOPS,
           "algo_GBps": byts / t / 1e9, "hbm_frac": byts / t / 1e9 / HBM_PEAK_GBS, "bound": "alu"}
    # VJP with respect to A: (nu-1)(nu-2)/2 recomputed forward steps plus nu-1
    # reverse steps (per step: Dout weight products, one FMA per CG entry,
    # two FMAs per (path, m1, m2) group)
    groups = sum(len({(int(a_), int(b_)) for a_, b_, _ in tb["cg_m"][tb["cg_ptr"][p]:tb["cg_ptr"][p + 1]]})
                 for p in range(len(tb["paths"])))
    G = torch.randn_like(A)
    gA = torch.empty_like(A)
    tv = time_calls(lambda: etp.etp_node_product_vjp(plan, A, W, G, gA, nu), reps)
    fv = float(n) * C * ((nu - 1) * (nu - 2) // 2 * f_step + (nu - 1) * (dout + 2 * nnz + 4 * groups))
    res.update({"vjp_ms": round(tv * 1e3, 4), "vjp_algo_TFLOPs": fv / tv / 1e12,
                "vjp_valu_frac": fv / tv / 1e12 / VALU_PEAK_TFLOPS})
    # the VJP with the weight gradient (per-node partials, then their ordered
    # sum over the nodes)
    ws = etp.node_product_wgrad_workspace(plan, n, nu)
    gW = torch.empty_like(W)
    tw = time_calls(lambda: etp.etp_node_product_vjp_wgrad(plan, A, W, G, gA, gW, nu, ws), reps)
    res.update({"vjp_wgrad_ms": round(tw * 1e3, 4)})
    return res


def next_ops(etp, reps):
    """The calls around the convolution (the 'next' rows), on the micro
    workload unless named."""
    import workloads
    p = Problem("micro")
    p.step(None, ("transpose", "fwd", "vjp"))
    d = {"radial": time_radial(etp, p, reps),
         "channel_mix": time_channel_mix(etp, p.plan, p.out, p.L, p.C, p.N, reps),
         "edge_forces": time_edge_forces(etp, p.g, p.gr, p.N, p.n_src, p.E, reps)}
    for name, (pos_np, box) in (("neighbor_list_water", workloads.water_positions(0)),
                                ("neighbor_list_diamond", workloads.diamond_positions(0))):
        d[name] = time_neighbor_list(etp, pos_np, box, 6.0, reps)
    d["edge_tp"] = time_edge_tp(etp, p.plan, p.L, p.C, p.E, (p.L + 1) ** 2, p.P, p.wl.Dout, p.vec, p.w, reps)
    del p
    p3 = Problem("micro3")
    p3.step(None, ("transpose", "fwd", "vjp"))
    d["radial_micro3"] = time_radial(etp, p3, reps)
    d["channel_mix_micro3"] = time_channel_mix(etp, p3.plan, p3.out, p3.L, p3.C, p3.N, reps)
    del p3
    # the mixing at the micro4 and diamond node counts and widths (its input
    # is a convolution output of that shape, drawn at random here)
    import torch
    for name, Lm, Cm, Nm in (("micro4", 4, 128, 1024), ("diamond", 3, 128, 32768)):
        plan = etp.etp_plan_create(Lm, Cm)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(Nm + Lm)
        conv = torch.randn(Nm, plan.dout_rows, Cm, generator=gen, device="cuda")
        d["channel_mix_" + name] = time_channel_mix(etp, plan, conv, Lm, Cm, Nm, reps)
        del conv
    for Lp, nu in ((3, 4), (4, 6)):
        d[f"node_product_l{Lp}_nu{nu}"] = time_node_product(etp, Lp, nu, reps)
    return d


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(p, budget_s=12.0):
    """The oracle, as it is, on the first R destination rows of the headline
    graph (R sized to about budget_s of host time), on the same inputs as the
    GPU run (copied back from the device); edges/s of transpose + fwd + VJP +
    VJP-of-VJP."""
    import oracle
    wl, L = p.wl, p.L
    # a few hundred rows at most: repeated passes fill the budget, and the
    # sample's per-edge arrays (copied to the host, widened to float64 by
    # the oracle) stay small
    rmax = min(wl.n_dst, 256)
    emax = int(wl.row_ptr[rmax])
    w = p.w[:emax].cpu().numpy()
    G = p.G[:rmax].cpu().numpy()
    ggx = p.ggx.cpu().numpy()
    x = p.x.float().cpu().numpy()
    if p.ggw_full is not None:
        ggw = p.ggw_full[:emax].cpu().numpy()
    else:
        ch0 = p.chunks[0]
        ggw = p.fill_ggw(0)[:min(emax, ch0["e1"] - ch0["e0"])].cpu().numpy()
        rmax = min(rmax, ch0["r1"])
        emax = int(wl.row_ptr[rmax])

    def run(R):
        rp = wl.row_ptr[:R + 1].copy()
        e1 = int(rp[-1])
        src, vec = wl.src[:e1], wl.vec[:e1]
        t0 = time.perf_counter()
        oracle.transpose(rp, src, wl.n)
        oracle.fwd(L, rp, src, vec, x, w[:e1])
        oracle.vjp(L, rp, src, vec, x, w[:e1], G[:R])
        oracle.vjp2(L, rp, src, vec, x, w[:e1], G[:R], ggx, ggw[:e1], wl.ggvec[:e1])
        return e1, time.perf_counter() - t0

    # time per edge from two probe sizes (each call also has a fixed cost:
    # CG tables, the source-side work over all nodes)
    r1, r2 = min(4, rmax), min(32, rmax)
    e_a, t_a = run(r1)
    e_b, t_b = run(r2)
    per_edge = max((t_b - t_a) / max(e_b - e_a, 1), 1e-9) if e_b > e_a else t_b / max(e_b, 1)
    fixed = max(t_a - per_edge * e_a, 0.0)
    R = int(min(rmax, max(r1, (budget_s - fixed) / per_edge / max(wl.E / wl.n_dst, 1))))
    e1, t = run(R)
    passes, e_tot, t_tot = 1, e1, t
    while t_tot < 0.8 * budget_s and passes < 64:
        e_k, t_k = run(R)
        passes, e_tot, t_tot = passes + 1, e_tot + e_k, t_tot + t_k
    return {"value": e_tot / t_tot, "unit": "edges/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"first {R} destination rows ({e1} edges) of the {p.name} graph, {passes} pass(es); "
                      f"transpose + fwd + VJP + VJP2 in float64 on the GPU run's inputs, {t_tot:.1f} s wall"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="diamond", choices=sorted(WORKLOADS))
    ap.add_argument("--configs", default="tiny,micro,micro3,micro4,water",
                    help="other workloads timed in the same run ('none' for none)")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bf16-feature run of the headline workload")
    ap.add_argument("--no-next", action="store_true", help="skip the calls around the convolution")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--bwd", default="auto", choices=("auto", "dst", "src"),
                    help="backward of the step: the workspace entry points with the library's choice per shape "
                         "(auto) or forced to walk each destination's in-edges (dst), or the entry points without "
                         "workspace (src); both forced formulations are timed beside it")
    ap.add_argument("--no-other-bwd", action="store_true", help="skip timing the forced backward formulations")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a kernel of known traffic "
                         "for scaling hardware byte counters)")
    a = ap.parse_args(argv)
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the convolution would shard by destination node with halo exchanges; "
              "that exchange is not built). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from equivariant_interatomic_potentials_amd import etp

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    print(f"[bench] {a.workload}: building inputs", file=sys.stderr, flush=True)
    if a.calib_copy_mib:
        n = a.calib_copy_mib * (1 << 20) // 4
        cs, cd = torch.ones(n, device="cuda"), torch.empty(n, device="cuda")
        cd.copy_(cs)
        torch.cuda.synchronize()
        del cs, cd
    p = Problem(a.workload, bwd=a.bwd)
    print(f"[bench] {a.workload}: E={p.E}, VJP-of-VJP in {len(p.chunks)} chunk(s); timing", file=sys.stderr,
          flush=True)
    t0 = time.perf_counter()
    per_op, ms_step = p.run(a.steps, a.warmup)
    timed_s = time.perf_counter() - t0
    rep, by, fl = p.report(per_op)
    N, E = p.N, p.E
    fwd_vjp = E / ((per_op["fwd"] + per_op["vjp"]) * 1e-3)
    t_roof = {op: max(by[op] / (HBM_PEAK_GBS * 1e9), fl[op] / (VALU_PEAK_TFLOPS * 1e12)) for op in OPS}
    fwd_vjp_roof = E / (t_roof["fwd"] + t_roof["vjp"])
    dom = max(("fwd", "vjp", "vjp2"), key=lambda o: per_op[o])
    roofline = roof(by[dom], fl[dom], per_op[dom] * 1e-3)
    roofline.update({"traffic": measured_traffic(a.workload, dom), "op": dom,
                     "basis": "compulsory bytes / FLOPs of the whole op (every kernel it launches), "
                              "HIP events around each call"})

    line = {
        "metric": METRIC, "value": fwd_vjp, "unit": "edges/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{a.workload}: {WORKLOADS[a.workload]}", "n_nodes": N, "n_edges": E,
                   "channels": p.C, "l_max": p.L, "x_storage": "f32",
                   "step": "csr_transpose + fwd + vjp + vjp2", "vjp2_chunks": len(p.chunks), "bwd": p.bwd},
        "value_is": "fwd+VJP edges/s = E / (t_fwd + t_vjp)",
        "fwd_edges_per_s": rep["fwd"]["edges_per_s"],
        "fwd_vjp_edges_per_s": fwd_vjp,
        "fwd_vjp_frac": round(fwd_vjp / fwd_vjp_roof, 4),
        "step_edges_per_s": E / (sum(per_op.values()) * 1e-3),
        "ops": rep,
        "roofline": roofline,
    }
    print(f"[bench] {a.workload} f32: fwd {per_op['fwd']:.3f} ms, vjp {per_op['vjp']:.3f} ms, "
          f"vjp2 {per_op['vjp2']:.3f} ms ({timed_s:.1f} s)", file=sys.stderr, flush=True)
    if not a.no_other_bwd:
        line["other_bwd"] = other_bwd(p, a.steps, a.warmup)
        for b, o in line["other_bwd"].items():
            print(f"[bench] {a.workload} backward forced {b}: vjp {o['vjp']['ms']:.3f} ms, "
                  f"vjp2 {o['vjp2']['ms']:.3f} ms", file=sys.stderr, flush=True)
    if not a.no_bf16 and p.L >= 1:
        pb = Problem(a.workload, bf16=True, shared=p.shared(), bwd=a.bwd)
        per_b, ms_b = pb.run(a.steps, a.warmup)
        rep_b, _, _ = pb.report(per_b)
        line["bf16_x"] = {"fwd_edges_per_s": rep_b["fwd"]["edges_per_s"],
                          "fwd_vjp_edges_per_s": E / ((per_b["fwd"] + per_b["vjp"]) * 1e-3),
                          "ms_per_step": ms_b, "ops": rep_b}
        print(f"[bench] {a.workload} bf16 x: fwd {per_b['fwd']:.3f} ms, vjp {per_b['vjp']:.3f} ms, "
              f"vjp2 {per_b['vjp2']:.3f} ms", file=sys.stderr, flush=True)
        del pb
    if not a.no_cpu:
        print("[bench] oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(p)
    shared_keys = p.shared()
    del p, shared_keys
    torch.cuda.empty_cache()
    names = [] if a.configs == "none" else [c for c in a.configs.split(",") if c and c != a.workload]
    if names:
        line["configs"] = {}
        for c in names:
            print(f"[bench] config {c}", file=sys.stderr, flush=True)
            line["configs"][c] = config_entry(c, a.steps, a.warmup, a.bwd)
    if not a.no_next:
        print("[bench] calls around the convolution", file=sys.stderr, flush=True)
        line["next_ops"] = next_ops(etp, a.steps)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
