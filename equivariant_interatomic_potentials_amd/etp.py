"""Thin Python binding of libetp (include/etp.h), same names as the C ABI.

Argument marshalling only: tensors are passed by device pointer
(``tensor.data_ptr()``), the stream is torch's current HIP stream unless
given, and every non-zero status raises ``EtpError``. All the computation
runs in libetp's HIP kernels; there is no fallback path -- importing this
module fails loudly if libetp.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libetp.so")

ETP_OK = 0
ETP_ERR_INVALID_ARGUMENT = 1
ETP_ERR_UNSUPPORTED = 2
ETP_ERR_WORKSPACE = 3
ETP_ERR_HIP = 4
ETP_ERR_ALLOC = 5
ETP_ERR_INTERNAL = 6
ETP_F32 = 0
ETP_BF16 = 1
ETP_FLAG_ACCUMULATE = 1
ETP_FLAG_VALIDATE = 2
ETP_FLAG_DST_PASS = 4
ETP_FLAG_SRC_PASS = 8

# every symbol include/etp.h declares
ABI_SYMBOLS = ("etp_plan_create", "etp_plan_destroy", "etp_plan_info", "etp_plan_describe", "etp_plan_tables",
               "etp_csr_transpose_workspace", "etp_csr_transpose", "etp_workspace_size", "etp_sh", "etp_edge_conv_fwd",
               "etp_edge_conv_fwd_radial", "etp_edge_conv_vjp_radial",
               "etp_edge_conv_vjp", "etp_edge_conv_vjp2", "etp_edge_conv_vjp2_radial", "etp_channel_mix",
               "etp_edge_forces",
               "etp_neighbor_workspace", "etp_neighbor_count", "etp_neighbor_fill", "etp_node_product", "etp_node_product_vjp", "etp_channel_mix_vjp",
               "etp_edge_tp_fwd", "etp_edge_tp_vjp", "etp_edge_tp_vjp2",
               "etp_csr_transpose_noalloc", "etp_edge_conv_vjp_ws", "etp_edge_conv_vjp2_ws",
               "etp_edge_conv_vjp_radial_wgrad", "etp_edge_conv_vjp2_radial_wgrad", "etp_channel_mix_ex", "etp_channel_mix_vjp_ex", "etp_channel_mix_wgrad", "etp_node_product_vjp_wgrad", "etp_node_product_wgrad_workspace",
               "etp_status_string", "etp_version")


class EtpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {etp_status_string(status)} (status {status})")


class etp_plan_desc(ctypes.Structure):
    _fields_ = [("l_max_in", ctypes.c_int32), ("l_max_sh", ctypes.c_int32), ("l_max_out", ctypes.c_int32),
                ("channels", ctypes.c_int32), ("x_dtype", ctypes.c_int32), ("n_paths", ctypes.c_int32),
                ("paths", ctypes.POINTER(ctypes.c_int32))]


class etp_graph(ctypes.Structure):
    _fields_ = [("n_dst", ctypes.c_int32), ("n_src", ctypes.c_int32), ("n_edges", ctypes.c_int64),
                ("row_ptr", ctypes.c_void_p), ("src", ctypes.c_void_p), ("src_ptr", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("perm_dst", ctypes.c_void_p)]


class etp_plan_info_t(ctypes.Structure):
    _fields_ = [("l_max", ctypes.c_int32), ("channels", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("n_paths", ctypes.c_int32), ("nnz", ctypes.c_int32), ("din_rows", ctypes.c_int32),
                ("dsh", ctypes.c_int32), ("dout_rows", ctypes.c_int32)]


def _hip_runtimes():
    """Distinct libamdhip64 files mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1]
                if "libamdhip64.so" in os.path.basename(path):
                    found.add(os.path.realpath(path))
    except OSError:
        pass
    return found


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run "
                          "`python -m equivariant_interatomic_potentials_amd.build`")
    # torch provides device memory and streams and ships its own HIP runtime
    # (same soname as the system one). Loading torch first makes libetp bind
    # to that runtime, so there is exactly one HIP runtime in the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(_LIB_PATH)
    rts = _hip_runtimes()
    if len(rts) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({sorted(rts)}); import torch before loading libetp")
    vp, st, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    sig = {
        "etp_plan_create": (st, [ctypes.POINTER(etp_plan_desc), ctypes.POINTER(vp)]),
        "etp_plan_destroy": (st, [vp]),
        "etp_plan_info": (st, [vp, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
                               ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                               ctypes.POINTER(ctypes.c_int32)]),
        "etp_plan_describe": (st, [vp, ctypes.POINTER(etp_plan_info_t)]),
        "etp_plan_tables": (st, [vp, vp, vp, vp, vp, vp]),
        "etp_csr_transpose_workspace": (st, [i32, ctypes.POINTER(ctypes.c_size_t)]),
        "etp_csr_transpose": (st, [ctypes.POINTER(etp_graph), vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "etp_csr_transpose_noalloc": (st, [ctypes.POINTER(etp_graph), vp, vp, vp, vp]),
        "etp_workspace_size": (st, [vp, i32, ctypes.POINTER(etp_graph), ctypes.POINTER(ctypes.c_size_t)]),
        "etp_sh": (st, [vp, i64, vp, vp, vp, vp]),
        "etp_edge_conv_fwd": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, vp, u32, vp]),
        "etp_edge_conv_fwd_radial": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, i32, vp, vp, u32, vp]),
        "etp_edge_conv_vjp_radial": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, i32, vp, vp, vp, vp, vp, u32,
                                          vp]),
        "etp_edge_conv_vjp": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, vp, vp, vp, vp, u32, vp]),
        "etp_edge_conv_vjp2_radial": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, u32, vp]),
        "etp_edge_conv_vjp2": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, u32, vp]),
        "etp_edge_conv_vjp_ws": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, vp, vp, vp, vp, u32, vp,
                                      ctypes.c_size_t, vp]),
        "etp_edge_conv_vjp_radial_wgrad": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                                vp, u32, vp, ctypes.c_size_t, vp]),
        "etp_edge_conv_vjp2_radial_wgrad": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                                 vp, vp, vp, vp, vp, u32, vp, ctypes.c_size_t, vp]),
        "etp_edge_conv_vjp2_ws": (st, [vp, ctypes.POINTER(etp_graph), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, u32, vp, ctypes.c_size_t, vp]),
        "etp_channel_mix": (st, [vp, i32, vp, vp, vp, u32, vp]),
        "etp_channel_mix_ex": (st, [vp, i32, vp, vp, i32, vp, u32, vp]),
        "etp_channel_mix_vjp_ex": (st, [vp, i32, vp, vp, i32, vp, u32, vp]),
        "etp_channel_mix_wgrad": (st, [vp, i32, vp, vp, vp, u32, vp, ctypes.c_size_t, vp]),
        "etp_node_product_vjp_wgrad": (st, [vp, i32, i32, vp, vp, vp, vp, vp, u32, vp, ctypes.c_size_t, vp]),
        "etp_node_product_wgrad_workspace": (st, [vp, i32, i32, vp]),
        "etp_edge_forces": (st, [ctypes.POINTER(etp_graph), vp, vp, u32, vp]),
        "etp_node_product": (st, [vp, i32, i32, vp, vp, vp, u32, vp]),
        "etp_channel_mix_vjp": (st, [vp, i32, vp, vp, vp, u32, vp]),
        "etp_node_product_vjp": (st, [vp, i32, i32, vp, vp, vp, vp, u32, vp]),
        "etp_edge_tp_fwd": (st, [vp, i64, vp, vp, vp, vp, u32, vp]),
        "etp_edge_tp_vjp": (st, [vp, i64, vp, vp, vp, vp, vp, vp, vp, u32, vp]),
        "etp_edge_tp_vjp2": (st, [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, u32, vp]),
        "etp_neighbor_workspace": (st, [i32, vp, ctypes.c_float, ctypes.POINTER(ctypes.c_size_t)]),
        "etp_neighbor_count": (st, [i32, vp, vp, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]),
        "etp_neighbor_fill": (st, [i32, vp, vp, ctypes.c_float, vp, i64, vp, vp, u32, vp, ctypes.c_size_t, vp]),
        "etp_status_string": (ctypes.c_char_p, [st]),
        "etp_version": (i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def _check(status: int, where: str):
    if status != ETP_OK:
        raise EtpError(status, where)


def _ptr(t, name, dtype=None, numel=None, optional=False):
    """Device pointer of a contiguous tensor (None -> NULL if optional)."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr() if t.numel() else None


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def etp_status_string(status: int) -> str:
    return lib.etp_status_string(status).decode()


def etp_version() -> int:
    return lib.etp_version()


class Plan:
    """An etp_plan_t handle (destroyed with the object)."""

    def __init__(self, handle: int):
        self.handle = handle
        info = etp_plan_info(self)
        self.L = info["l_max"]
        self.C = info["channels"]
        self.x_dtype = info["x_dtype"]
        self.P = info["n_paths"]
        self.nnz = info["nnz"]
        self.din_rows = info["din_rows"]
        self.dsh = info["dsh"]
        self.dout_rows = info["dout_rows"]

    def __del__(self):
        # at interpreter exit the module's globals may already be gone
        if getattr(self, "handle", None) and lib is not None:
            lib.etp_plan_destroy(self.handle)
            self.handle = None


def etp_plan_create(l_max, channels: int, x_dtype: int = ETP_F32, paths=None) -> Plan:
    """l_max: int or (l_max_in, l_max_sh, l_max_out); paths: optional host [P, 3] int array."""
    lin, lsh, lout = (l_max, l_max, l_max) if isinstance(l_max, int) else tuple(l_max)
    d = etp_plan_desc(lin, lsh, lout, channels, x_dtype, 0, None)
    keep = None
    if paths is not None:
        keep = np.ascontiguousarray(paths, dtype=np.int32).reshape(-1, 3)
        d.n_paths = keep.shape[0]
        d.paths = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    h = ctypes.c_void_p()
    _check(lib.etp_plan_create(ctypes.byref(d), ctypes.byref(h)), "etp_plan_create")
    return Plan(h.value)


def etp_plan_destroy(plan: Plan):
    if plan.handle:
        _check(lib.etp_plan_destroy(plan.handle), "etp_plan_destroy")
        plan.handle = None


def etp_plan_describe(plan: Plan) -> dict:
    info = etp_plan_info_t()
    _check(lib.etp_plan_describe(plan.handle, ctypes.byref(info)), "etp_plan_describe")
    return {k: getattr(info, k) for k, _ in etp_plan_info_t._fields_}


def etp_plan_info(plan: Plan) -> dict:
    """n_paths, din, dsh, dout (floats per node / SH per edge) and nnz, plus the
    per-channel row counts and the plan's l_max, channels and dtype."""
    n_paths, nnz = ctypes.c_int32(), ctypes.c_int32()
    din, dsh, dout = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib.etp_plan_info(plan.handle, ctypes.byref(n_paths), ctypes.byref(din), ctypes.byref(dsh),
                             ctypes.byref(dout), ctypes.byref(nnz)), "etp_plan_info")
    d = etp_plan_describe(plan)
    d.update(n_paths=n_paths.value, nnz=nnz.value, din=din.value, dsh=dsh.value, dout=dout.value)
    return d


def etp_plan_tables(plan: Plan) -> dict:
    info = etp_plan_info(plan)
    P, nnz = info["n_paths"], info["nnz"]
    paths = np.zeros((P, 3), np.int32)
    out_off = np.zeros(P + 1, np.int32)
    cg_ptr = np.zeros(P + 1, np.int32)
    cg_m = np.zeros((nnz, 3), np.int8)
    cg_val = np.zeros(nnz, np.float32)
    _check(lib.etp_plan_tables(plan.handle, paths.ctypes.data, out_off.ctypes.data, cg_ptr.ctypes.data,
                               cg_m.ctypes.data, cg_val.ctypes.data), "etp_plan_tables")
    return dict(paths=paths, out_off=out_off, cg_ptr=cg_ptr, cg_m=cg_m, cg_val=cg_val)


class Graph:
    """Device CSR (+ optional transpose) with the etp_graph struct."""

    def __init__(self, n_dst, n_src, row_ptr, src, src_ptr=None, perm=None, perm_dst=None, n_edges=None):
        self.n_dst, self.n_src = int(n_dst), int(n_src)
        self.n_edges = int(src.numel()) if n_edges is None else int(n_edges)
        self.row_ptr, self.src = row_ptr, src
        self.src_ptr, self.perm, self.perm_dst = src_ptr, perm, perm_dst

    def struct(self) -> etp_graph:
        import torch
        g = etp_graph()
        g.n_dst, g.n_src, g.n_edges = self.n_dst, self.n_src, self.n_edges
        g.row_ptr = _ptr(self.row_ptr, "row_ptr", torch.int32, self.n_dst + 1, optional=True)
        g.src = _ptr(self.src, "src", torch.int32, self.n_edges, optional=True)
        g.src_ptr = _ptr(self.src_ptr, "src_ptr", torch.int32, self.n_src + 1, optional=True)
        g.perm = _ptr(self.perm, "perm", torch.int32, self.n_edges, optional=True)
        g.perm_dst = _ptr(self.perm_dst, "perm_dst", torch.int32, self.n_edges, optional=True)
        return g


def etp_csr_transpose_workspace(n_src: int) -> int:
    b = ctypes.c_size_t()
    _check(lib.etp_csr_transpose_workspace(n_src, ctypes.byref(b)), "etp_csr_transpose_workspace")
    return b.value


ETP_OP_FWD, ETP_OP_VJP, ETP_OP_VJP2, ETP_OP_TRANSPOSE, ETP_OP_VJP_WS, ETP_OP_VJP2_WS = 0, 1, 2, 3, 4, 5
ETP_OP_RADIAL_WGRAD = 6
ETP_OP_MIX_WGRAD = 7


def etp_workspace_size(plan: Plan, op: int, graph: Graph) -> int:
    b = ctypes.c_size_t()
    g = graph.struct()
    _check(lib.etp_workspace_size(plan.handle, op, ctypes.byref(g), ctypes.byref(b)), "etp_workspace_size")
    return b.value


def etp_csr_transpose(graph: Graph, src_ptr, perm, perm_dst, ws, stream=None):
    import torch
    g = graph.struct()
    _check(lib.etp_csr_transpose(ctypes.byref(g), _ptr(src_ptr, "src_ptr", torch.int32, graph.n_src + 1),
                                 _ptr(perm, "perm", torch.int32, graph.n_edges, optional=True),
                                 _ptr(perm_dst, "perm_dst", torch.int32, graph.n_edges, optional=True),
                                 _ptr(ws, "ws", optional=True), ws.numel() * ws.element_size() if ws is not None else 0,
                                 _stream(stream)), "etp_csr_transpose")


ETP_NOALLOC_MAX_SOURCES = 1 << 20


def etp_csr_transpose_noalloc(graph: Graph, src_ptr, perm, perm_dst, stream=None):
    """etp_csr_transpose with the library's fixed device workspace (allocates nothing)."""
    import torch
    g = graph.struct()
    _check(lib.etp_csr_transpose_noalloc(ctypes.byref(g), _ptr(src_ptr, "src_ptr", torch.int32, graph.n_src + 1),
                                         _ptr(perm, "perm", torch.int32, graph.n_edges, optional=True),
                                         _ptr(perm_dst, "perm_dst", torch.int32, graph.n_edges, optional=True),
                                         _stream(stream)), "etp_csr_transpose_noalloc")


def etp_sh(plan: Plan, vec, Y, dY=None, stream=None):
    import torch
    n = vec.numel() // 3
    _check(lib.etp_sh(plan.handle, n, _ptr(vec, "vec", torch.float32, 3 * n, optional=True),
                      _ptr(Y, "Y", torch.float32, n * plan.dsh, optional=True),
                      _ptr(dY, "dY", torch.float32, 3 * n * plan.dsh, optional=True), _stream(stream)), "etp_sh")


def _xdtype(plan):
    import torch
    return torch.bfloat16 if plan.x_dtype == ETP_BF16 else torch.float32


def etp_edge_conv_fwd(plan: Plan, graph: Graph, vec, x, w, out, flags: int = 0, stream=None):
    import torch
    E, C = graph.n_edges, plan.C
    g = graph.struct()
    _check(lib.etp_edge_conv_fwd(plan.handle, ctypes.byref(g),
                                 _ptr(vec, "vec", torch.float32, 3 * E, optional=True),
                                 _ptr(x, "x", _xdtype(plan), graph.n_src * plan.din_rows * C, optional=True),
                                 _ptr(w, "w", torch.float32, E * plan.P * C, optional=True),
                                 _ptr(out, "out", torch.float32, graph.n_dst * plan.dout_rows * C, optional=True),
                                 flags, _stream(stream)), "etp_edge_conv_fwd")


def etp_edge_conv_fwd_radial(plan: Plan, graph: Graph, vec, x, h, Wr, out, flags: int = 0, stream=None):
    """The forward with w = h @ Wr formed in the kernel: h [E, K], Wr [K, P, C]."""
    import torch
    E, C = graph.n_edges, plan.C
    K = int(Wr.shape[0]) if Wr is not None else 0
    g = graph.struct()
    _check(lib.etp_edge_conv_fwd_radial(plan.handle, ctypes.byref(g),
                                        _ptr(vec, "vec", torch.float32, 3 * E, optional=True),
                                        _ptr(x, "x", _xdtype(plan), graph.n_src * plan.din_rows * C, optional=True),
                                        _ptr(h, "h", torch.float32, E * K, optional=True), K,
                                        _ptr(Wr, "Wr", torch.float32, K * plan.P * C, optional=True),
                                        _ptr(out, "out", torch.float32, graph.n_dst * plan.dout_rows * C, optional=True),
                                        flags, _stream(stream)), "etp_edge_conv_fwd_radial")


def etp_edge_conv_vjp_radial(plan: Plan, graph: Graph, vec, x, h, Wr, grad_out, grad_x=None, grad_h=None,
                             grad_vec=None, flags: int = 0, stream=None):
    """VJP of etp_edge_conv_fwd_radial: grad_x, grad_h [E, K], grad_vec (each optional)."""
    import torch
    E, C = graph.n_edges, plan.C
    K = int(Wr.shape[0]) if Wr is not None else 0
    g = graph.struct()
    _check(lib.etp_edge_conv_vjp_radial(
        plan.handle, ctypes.byref(g),
        _ptr(vec, "vec", torch.float32, 3 * E, optional=True),
        _ptr(x, "x", _xdtype(plan), graph.n_src * plan.din_rows * C, optional=True),
        _ptr(h, "h", torch.float32, E * K, optional=True), K,
        _ptr(Wr, "Wr", torch.float32, K * plan.P * C, optional=True),
        _ptr(grad_out, "grad_out", torch.float32, graph.n_dst * plan.dout_rows * C, optional=True),
        _ptr(grad_x, "grad_x", torch.float32, graph.n_src * plan.din_rows * C, optional=True),
        _ptr(grad_h, "grad_h", torch.float32, E * K, optional=True),
        _ptr(grad_vec, "grad_vec", torch.float32, 3 * E, optional=True),
        flags, _stream(stream)), "etp_edge_conv_vjp_radial")


def etp_edge_conv_vjp2_radial(plan: Plan, graph: Graph, vec, x, h, Wr, grad_out, gg_x=None, gg_h=None, gg_vec=None,
                              d_x=None, d_h=None, d_vec=None, d_grad_out=None, flags: int = 0, stream=None):
    """VJP of etp_edge_conv_vjp_radial: d_x, d_h [E, K], d_vec, d_grad_out (each optional)."""
    import torch
    E, C = graph.n_edges, plan.C
    K = int(Wr.shape[0]) if Wr is not None else 0
    f32 = torch.float32
    nx, no = graph.n_src * plan.din_rows * C, graph.n_dst * plan.dout_rows * C
    g = graph.struct()
    _check(lib.etp_edge_conv_vjp2_radial(
        plan.handle, ctypes.byref(g),
        _ptr(vec, "vec", f32, 3 * E, optional=True),
        _ptr(x, "x", _xdtype(plan), nx, optional=True),
        _ptr(h, "h", f32, E * K, optional=True), K,
        _ptr(Wr, "Wr", f32, K * plan.P * C, optional=True),
        _ptr(grad_out, "grad_out", f32, no, optional=True),
        _ptr(gg_x, "gg_x", f32, nx, optional=True),
        _ptr(gg_h, "gg_h", f32, E * K, optional=True),
        _ptr(gg_vec, "gg_vec", f32, 3 * E, optional=True),
        _ptr(d_x, "d_x", f32, nx, optional=True),
        _ptr(d_h, "d_h", f32, E * K, optional=True),
        _ptr(d_vec, "d_vec", f32, 3 * E, optional=True),
        _ptr(d_grad_out, "d_grad_out", f32, no, optional=True),
        flags, _stream(stream)), "etp_edge_conv_vjp2_radial")


def etp_edge_conv_vjp_radial_wgrad(plan: Plan, graph: Graph, vec, x, h, Wr, grad_out, grad_x=None, grad_h=None,
                                   grad_vec=None, grad_Wr=None, ws=None, flags: int = 0, stream=None):
    """etp_edge_conv_vjp_radial plus grad_Wr [K, P, C]; ws: etp_workspace_size(plan, ETP_OP_RADIAL_WGRAD, graph)
    bytes."""
    import torch
    E, C = graph.n_edges, plan.C
    K = int(Wr.shape[0]) if Wr is not None else 0
    f32 = torch.float32
    g = graph.struct()
    wp, wb = _ws(ws)
    _check(lib.etp_edge_conv_vjp_radial_wgrad(
        plan.handle, ctypes.byref(g),
        _ptr(vec, "vec", f32, 3 * E, optional=True),
        _ptr(x, "x", _xdtype(plan), graph.n_src * plan.din_rows * C, optional=True),
        _ptr(h, "h", f32, E * K, optional=True), K,
        _ptr(Wr, "Wr", f32, K * plan.P * C, optional=True),
        _ptr(grad_out, "grad_out", f32, graph.n_dst * plan.dout_rows * C, optional=True),
        _ptr(grad_x, "grad_x", f32, graph.n_src * plan.din_rows * C, optional=True),
        _ptr(grad_h, "grad_h", f32, E * K, optional=True),
        _ptr(grad_vec, "grad_vec", f32, 3 * E, optional=True),
        _ptr(grad_Wr, "grad_Wr", f32, K * plan.P * C, optional=True),
        flags, wp, wb, _stream(stream)), "etp_edge_conv_vjp_radial_wgrad")


def etp_edge_conv_vjp2_radial_wgrad(plan: Plan, graph: Graph, vec, x, h, Wr, grad_out, gg_x=None, gg_h=None,
                                    gg_vec=None, d_x=None, d_h=None, d_vec=None, d_grad_out=None, d_Wr=None,
                                    ws=None, flags: int = 0, stream=None):
    """etp_edge_conv_vjp2_radial plus d_Wr [K, P, C]; ws as for etp_edge_conv_vjp_radial_wgrad."""
    import torch
    E, C = graph.n_edges, plan.C
    K = int(Wr.shape[0]) if Wr is not None else 0
    f32 = torch.float32
    nx, no = graph.n_src * plan.din_rows * C, graph.n_dst * plan.dout_rows * C
    g = graph.struct()
    wp, wb = _ws(ws)
    _check(lib.etp_edge_conv_vjp2_radial_wgrad(
        plan.handle, ctypes.byref(g),
        _ptr(vec, "vec", f32, 3 * E, optional=True),
        _ptr(x, "x", _xdtype(plan), nx, optional=True),
        _ptr(h, "h", f32, E * K, optional=True), K,
        _ptr(Wr, "Wr", f32, K * plan.P * C, optional=True),
        _ptr(grad_out, "grad_out", f32, no, optional=True),
        _ptr(gg_x, "gg_x", f32, nx, optional=True),
        _ptr(gg_h, "gg_h", f32, E * K, optional=True),
        _ptr(gg_vec, "gg_vec", f32, 3 * E, optional=True),
        _ptr(d_x, "d_x", f32, nx, optional=True),
        _ptr(d_h, "d_h", f32, E * K, optional=True),
        _ptr(d_vec, "d_vec", f32, 3 * E, optional=True),
        _ptr(d_grad_out, "d_grad_out", f32, no, optional=True),
        _ptr(d_Wr, "d_Wr", f32, K * plan.P * C, optional=True),
        flags, wp, wb, _stream(stream)), "etp_edge_conv_vjp2_radial_wgrad")


def etp_edge_conv_vjp(plan: Plan, graph: Graph, vec, x, w, grad_out, grad_x=None, grad_w=None, grad_vec=None,
                      flags: int = 0, stream=None):
    import torch
    E, C = graph.n_edges, plan.C
    f32 = torch.float32
    g = graph.struct()
    _check(lib.etp_edge_conv_vjp(plan.handle, ctypes.byref(g),
                                 _ptr(vec, "vec", f32, 3 * E, optional=True),
                                 _ptr(x, "x", _xdtype(plan), graph.n_src * plan.din_rows * C, optional=True),
                                 _ptr(w, "w", f32, E * plan.P * C, optional=True),
                                 _ptr(grad_out, "grad_out", f32, graph.n_dst * plan.dout_rows * C, optional=True),
                                 _ptr(grad_x, "grad_x", f32, graph.n_src * plan.din_rows * C, optional=True),
                                 _ptr(grad_w, "grad_w", f32, E * plan.P * C, optional=True),
                                 _ptr(grad_vec, "grad_vec", f32, 3 * E, optional=True),
                                 flags, _stream(stream)), "etp_edge_conv_vjp")


def etp_edge_conv_vjp2(plan: Plan, graph: Graph, vec, x, w, grad_out, gg_x=None, gg_w=None, gg_vec=None,
                       d_x=None, d_w=None, d_vec=None, d_grad_out=None, flags: int = 0, stream=None):
    import torch
    E, C = graph.n_edges, plan.C
    f32 = torch.float32
    nx, nw, no = graph.n_src * plan.din_rows * C, E * plan.P * C, graph.n_dst * plan.dout_rows * C
    g = graph.struct()
    _check(lib.etp_edge_conv_vjp2(plan.handle, ctypes.byref(g),
                                  _ptr(vec, "vec", f32, 3 * E, optional=True),
                                  _ptr(x, "x", _xdtype(plan), nx, optional=True),
                                  _ptr(w, "w", f32, nw, optional=True),
                                  _ptr(grad_out, "grad_out", f32, no, optional=True),
                                  _ptr(gg_x, "gg_x", f32, nx, optional=True),
                                  _ptr(gg_w, "gg_w", f32, nw, optional=True),
                                  _ptr(gg_vec, "gg_vec", f32, 3 * E, optional=True),
                                  _ptr(d_x, "d_x", f32, nx, optional=True),
                                  _ptr(d_w, "d_w", f32, nw, optional=True),
                                  _ptr(d_vec, "d_vec", f32, 3 * E, optional=True),
                                  _ptr(d_grad_out, "d_grad_out", f32, no, optional=True),
                                  flags, _stream(stream)), "etp_edge_conv_vjp2")


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws, "ws"), ws.numel() * ws.element_size())


def etp_edge_conv_vjp_ws(plan: Plan, graph: Graph, vec, x, w, grad_out, grad_x=None, grad_w=None, grad_vec=None,
                         ws=None, flags: int = 0, stream=None):
    """The VJP over each destination's in-edges; ws: device buffer of at least
    etp_workspace_size(plan, ETP_OP_VJP_WS, graph) bytes when grad_x is wanted."""
    import torch
    E, C = graph.n_edges, plan.C
    f32 = torch.float32
    g = graph.struct()
    wp, wb = _ws(ws)
    _check(lib.etp_edge_conv_vjp_ws(plan.handle, ctypes.byref(g),
                                    _ptr(vec, "vec", f32, 3 * E, optional=True),
                                    _ptr(x, "x", _xdtype(plan), graph.n_src * plan.din_rows * C, optional=True),
                                    _ptr(w, "w", f32, E * plan.P * C, optional=True),
                                    _ptr(grad_out, "grad_out", f32, graph.n_dst * plan.dout_rows * C, optional=True),
                                    _ptr(grad_x, "grad_x", f32, graph.n_src * plan.din_rows * C, optional=True),
                                    _ptr(grad_w, "grad_w", f32, E * plan.P * C, optional=True),
                                    _ptr(grad_vec, "grad_vec", f32, 3 * E, optional=True),
                                    flags, wp, wb, _stream(stream)), "etp_edge_conv_vjp_ws")


def etp_edge_conv_vjp2_ws(plan: Plan, graph: Graph, vec, x, w, grad_out, gg_x=None, gg_w=None, gg_vec=None,
                          d_x=None, d_w=None, d_vec=None, d_grad_out=None, ws=None, flags: int = 0, stream=None):
    """The VJP-of-VJP over each destination's in-edges; ws as for etp_edge_conv_vjp_ws (needed for d_x)."""
    import torch
    E, C = graph.n_edges, plan.C
    f32 = torch.float32
    nx, nw, no = graph.n_src * plan.din_rows * C, E * plan.P * C, graph.n_dst * plan.dout_rows * C
    g = graph.struct()
    wp, wb = _ws(ws)
    _check(lib.etp_edge_conv_vjp2_ws(plan.handle, ctypes.byref(g),
                                     _ptr(vec, "vec", f32, 3 * E, optional=True),
                                     _ptr(x, "x", _xdtype(plan), nx, optional=True),
                                     _ptr(w, "w", f32, nw, optional=True),
                                     _ptr(grad_out, "grad_out", f32, no, optional=True),
                                     _ptr(gg_x, "gg_x", f32, nx, optional=True),
                                     _ptr(gg_w, "gg_w", f32, nw, optional=True),
                                     _ptr(gg_vec, "gg_vec", f32, 3 * E, optional=True),
                                     _ptr(d_x, "d_x", f32, nx, optional=True),
                                     _ptr(d_w, "d_w", f32, nw, optional=True),
                                     _ptr(d_vec, "d_vec", f32, 3 * E, optional=True),
                                     _ptr(d_grad_out, "d_grad_out", f32, no, optional=True),
                                     flags, wp, wb, _stream(stream)), "etp_edge_conv_vjp2_ws")


def bwd_workspace(plan: Plan, graph: Graph, op: int = None):
    """A device workspace for etp_edge_conv_vjp_ws / _vjp2_ws (torch uint8 tensor, 256-byte aligned)."""
    import torch
    n = etp_workspace_size(plan, ETP_OP_VJP_WS if op is None else op, graph)
    return torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")


def mix_rows(plan: Plan):
    """Paths per output order l = 0..l_max (W_l has mix_rows[l] * C rows), from the plan's table."""
    t = etp_plan_tables(plan)
    l3 = t["paths"][:, 2]
    return [int((l3 == l).sum()) for l in range(plan.L + 1)]


def etp_channel_mix(plan: Plan, inp, W, out, flags: int = 0, stream=None):
    """out[n, (l_max+1)^2, C] = per-order channel mixing of the convolution output inp[n, dout_rows, C];
    W = W_0, W_1, ... back to back (W_l: [mix_rows[l] * C, C])."""
    import torch
    C = plan.C
    n = inp.shape[0] if inp is not None else 0
    nw = sum(mix_rows(plan)) * C * C
    _check(lib.etp_channel_mix(plan.handle, n, _ptr(inp, "in", torch.float32, n * plan.dout_rows * C, optional=True),
                               _ptr(W, "W", torch.float32, nw, optional=True),
                               _ptr(out, "out", torch.float32, n * (plan.L + 1) ** 2 * C, optional=True),
                               flags, _stream(stream)), "etp_channel_mix")


def etp_channel_mix_ex(plan: Plan, inp, W, out, flags: int = 0, stream=None):
    """etp_channel_mix with W in fp32 or bf16 (its torch dtype picks)."""
    import torch
    C = plan.C
    n = inp.shape[0] if inp is not None else 0
    nw = sum(mix_rows(plan)) * C * C
    bf = W is not None and W.dtype == torch.bfloat16
    _check(lib.etp_channel_mix_ex(plan.handle, n,
                                  _ptr(inp, "in", torch.float32, n * plan.dout_rows * C, optional=True),
                                  _ptr(W, "W", torch.bfloat16 if bf else torch.float32, nw, optional=True),
                                  ETP_BF16 if bf else ETP_F32,
                                  _ptr(out, "out", torch.float32, n * (plan.L + 1) ** 2 * C, optional=True),
                                  flags, _stream(stream)), "etp_channel_mix_ex")


def etp_channel_mix_vjp(plan: Plan, grad_y, W, grad_in, flags: int = 0, stream=None):
    """grad_in[n, Dout, C] = the transposed mixing of grad_y[n, (L+1)^2, C]."""
    import torch
    n = grad_y.shape[0]
    C = plan.C
    _check(lib.etp_channel_mix_vjp(plan.handle, n,
                                   _ptr(grad_y, "grad_y", torch.float32, n * (plan.L + 1) ** 2 * C, optional=True),
                                   _ptr(W, "W", torch.float32, sum(mix_rows(plan)) * C * C, optional=True),
                                   _ptr(grad_in, "grad_in", torch.float32, n * plan.dout_rows * C, optional=True),
                                   flags, _stream(stream)), "etp_channel_mix_vjp")


def etp_channel_mix_vjp_ex(plan: Plan, grad_y, W, grad_in, flags: int = 0, stream=None):
    """etp_channel_mix_vjp with W in fp32 or bf16 (its torch dtype picks)."""
    import torch
    n = grad_y.shape[0] if grad_y is not None else 0
    C = plan.C
    bf = W is not None and W.dtype == torch.bfloat16
    _check(lib.etp_channel_mix_vjp_ex(plan.handle, n,
                                      _ptr(grad_y, "grad_y", torch.float32, n * (plan.L + 1) ** 2 * C, optional=True),
                                      _ptr(W, "W", torch.bfloat16 if bf else torch.float32,
                                           sum(mix_rows(plan)) * C * C, optional=True),
                                      ETP_BF16 if bf else ETP_F32,
                                      _ptr(grad_in, "grad_in", torch.float32, n * plan.dout_rows * C, optional=True),
                                      flags, _stream(stream)), "etp_channel_mix_vjp_ex")


def mix_wgrad_workspace(plan: Plan, n: int):
    """A device workspace for etp_channel_mix_wgrad on n nodes (None when it does not split)."""
    import torch
    g = etp_graph()
    g.n_dst, g.n_src, g.n_edges = n, 0, 0  # the size query reads only the counts
    b = ctypes.c_size_t()
    _check(lib.etp_workspace_size(plan.handle, ETP_OP_MIX_WGRAD, ctypes.byref(g), ctypes.byref(b)),
           "etp_workspace_size")
    return torch.empty(b.value, dtype=torch.uint8, device="cuda") if b.value else None


def etp_channel_mix_wgrad(plan: Plan, inp, grad_y, grad_W, ws=None, flags: int = 0, stream=None):
    """grad_W (the layout of W) = per path, the sum over nodes and components of
    the input block times the cotangent row; ws from mix_wgrad_workspace."""
    import torch
    n = inp.shape[0] if inp is not None else 0
    C = plan.C
    wp, wb = _ws(ws)
    _check(lib.etp_channel_mix_wgrad(plan.handle, n,
                                     _ptr(inp, "in", torch.float32, n * plan.dout_rows * C, optional=True),
                                     _ptr(grad_y, "grad_y", torch.float32, n * (plan.L + 1) ** 2 * C, optional=True),
                                     _ptr(grad_W, "grad_W", torch.float32, sum(mix_rows(plan)) * C * C),
                                     flags, wp, wb, _stream(stream)), "etp_channel_mix_wgrad")


def etp_edge_forces(graph: Graph, grad_vec, forces, flags: int = 0, stream=None):
    """forces[max(n_dst, n_src), 3] = sum over in-edges of grad_vec - sum over out-edges (needs the transpose)."""
    import torch
    E = graph.n_edges
    n = max(graph.n_dst, graph.n_src)
    g = graph.struct()
    _check(lib.etp_edge_forces(ctypes.byref(g), _ptr(grad_vec, "grad_vec", torch.float32, 3 * E, optional=True),
                               _ptr(forces, "forces", torch.float32, 3 * n, optional=True), flags, _stream(stream)),
           "etp_edge_forces")


def etp_node_product(plan: Plan, A, W, out, corr_order: int, flags: int = 0, stream=None):
    """out[n, (L+1)^2, C] = B_1 + ... + B_nu, B_1 = A, B_{k+1} = sum_p W[k-1, p] * CG_p(B_k, A)."""
    import torch
    n = A.shape[0]
    D, C = plan.din_rows, plan.C
    _check(lib.etp_node_product(plan.handle, n, corr_order, _ptr(A, "A", torch.float32, n * D * C, optional=True),
                                _ptr(W, "W", torch.float32, (corr_order - 1) * plan.P * C, optional=True),
                                _ptr(out, "out", torch.float32, n * D * C, optional=True), flags,
                                _stream(stream)), "etp_node_product")


def etp_node_product_vjp(plan: Plan, A, W, grad_out, grad_A, corr_order: int, flags: int = 0, stream=None):
    """grad_A = d<grad_out, node_product(A)>/dA."""
    import torch
    n = A.shape[0]
    D, C = plan.din_rows, plan.C
    f32 = torch.float32
    _check(lib.etp_node_product_vjp(plan.handle, n, corr_order, _ptr(A, "A", f32, n * D * C, optional=True),
                                    _ptr(W, "W", f32, (corr_order - 1) * plan.P * C, optional=True),
                                    _ptr(grad_out, "grad_out", f32, n * D * C, optional=True),
                                    _ptr(grad_A, "grad_A", f32, n * D * C, optional=True), flags, _stream(stream)),
           "etp_node_product_vjp")


def node_product_wgrad_workspace(plan: Plan, n: int, corr_order: int):
    """A device workspace for etp_node_product_vjp_wgrad on n nodes."""
    import torch
    b = ctypes.c_size_t()
    _check(lib.etp_node_product_wgrad_workspace(plan.handle, n, corr_order, ctypes.byref(b)),
           "etp_node_product_wgrad_workspace")
    return torch.empty(max(b.value, 16), dtype=torch.uint8, device="cuda")


def etp_node_product_vjp_wgrad(plan: Plan, A, W, grad_out, grad_A, grad_W, corr_order: int, ws, flags: int = 0,
                               stream=None):
    """grad_A (may be None) and grad_W [corr_order-1, P, C] of <grad_out, etp_node_product(A, W)>."""
    import torch
    f32 = torch.float32
    n = A.shape[0] if A is not None else 0
    D = (plan.L + 1) ** 2
    C = plan.C
    P = len(etp_plan_tables(plan)["paths"])
    wp, wb = _ws(ws)
    _check(lib.etp_node_product_vjp_wgrad(plan.handle, n, corr_order, _ptr(A, "A", f32, n * D * C, optional=True),
                                          _ptr(W, "W", f32, (corr_order - 1) * P * C, optional=True),
                                          _ptr(grad_out, "grad_out", f32, n * D * C, optional=True),
                                          _ptr(grad_A, "grad_A", f32, n * D * C, optional=True),
                                          _ptr(grad_W, "grad_W", f32, (corr_order - 1) * P * C),
                                          flags, wp, wb, _stream(stream)), "etp_node_product_vjp_wgrad")


def etp_edge_tp_fwd(plan: Plan, vec, V, w, out, flags: int = 0, stream=None):
    """Edge-local tensor product: out[E, Dout, C] (no destination sum)."""
    import torch
    E, C = vec.numel() // 3, plan.C
    _check(lib.etp_edge_tp_fwd(plan.handle, E, _ptr(vec, "vec", torch.float32, 3 * E, optional=True),
                               _ptr(V, "V", torch.float32, E * plan.din_rows * C, optional=True),
                               _ptr(w, "w", torch.float32, E * plan.P * C, optional=True),
                               _ptr(out, "out", torch.float32, E * plan.dout_rows * C, optional=True), flags,
                               _stream(stream)), "etp_edge_tp_fwd")


def etp_edge_tp_vjp(plan: Plan, vec, V, w, grad_out, grad_V=None, grad_w=None, grad_vec=None, flags: int = 0,
                    stream=None):
    import torch
    E, C = vec.numel() // 3, plan.C
    f32 = torch.float32
    _check(lib.etp_edge_tp_vjp(plan.handle, E, _ptr(vec, "vec", f32, 3 * E, optional=True),
                               _ptr(V, "V", f32, E * plan.din_rows * C, optional=True),
                               _ptr(w, "w", f32, E * plan.P * C, optional=True),
                               _ptr(grad_out, "grad_out", f32, E * plan.dout_rows * C, optional=True),
                               _ptr(grad_V, "grad_V", f32, E * plan.din_rows * C, optional=True),
                               _ptr(grad_w, "grad_w", f32, E * plan.P * C, optional=True),
                               _ptr(grad_vec, "grad_vec", f32, 3 * E, optional=True), flags, _stream(stream)),
           "etp_edge_tp_vjp")


def etp_edge_tp_vjp2(plan: Plan, vec, V, w, grad_out, gg_V=None, gg_w=None, gg_vec=None, d_V=None, d_w=None,
                     d_vec=None, d_grad_out=None, flags: int = 0, stream=None):
    import torch
    E, C = vec.numel() // 3, plan.C
    f32 = torch.float32
    nv, nw, no = E * plan.din_rows * C, E * plan.P * C, E * plan.dout_rows * C
    _check(lib.etp_edge_tp_vjp2(plan.handle, E, _ptr(vec, "vec", f32, 3 * E, optional=True),
                                _ptr(V, "V", f32, nv, optional=True), _ptr(w, "w", f32, nw, optional=True),
                                _ptr(grad_out, "grad_out", f32, no, optional=True),
                                _ptr(gg_V, "gg_V", f32, nv, optional=True), _ptr(gg_w, "gg_w", f32, nw, optional=True),
                                _ptr(gg_vec, "gg_vec", f32, 3 * E, optional=True),
                                _ptr(d_V, "d_V", f32, nv, optional=True), _ptr(d_w, "d_w", f32, nw, optional=True),
                                _ptr(d_vec, "d_vec", f32, 3 * E, optional=True),
                                _ptr(d_grad_out, "d_grad_out", f32, no, optional=True), flags, _stream(stream)),
           "etp_edge_tp_vjp2")


def _box3(box):
    """Box sides as a HOST float[3] (kept alive by the caller)."""
    import numpy as np
    return np.ascontiguousarray(np.broadcast_to(np.asarray(box, np.float32), (3,)))


def etp_neighbor_workspace(n_atoms: int, box, cutoff: float) -> int:
    b = ctypes.c_size_t()
    bx = _box3(box)
    _check(lib.etp_neighbor_workspace(n_atoms, bx.ctypes.data, float(cutoff), ctypes.byref(b)),
           "etp_neighbor_workspace")
    return b.value


def etp_neighbor_count(pos, box, cutoff: float, row_ptr, ws, stream=None):
    """row_ptr[n+1] of the periodic neighbour list of pos[n, 3] (float32 cutoff decision)."""
    import torch
    n = pos.shape[0]
    bx = _box3(box)
    _check(lib.etp_neighbor_count(n, _ptr(pos, "pos", torch.float32, 3 * n, optional=True), bx.ctypes.data,
                                  float(cutoff), _ptr(row_ptr, "row_ptr", torch.int32, n + 1),
                                  _ptr(ws, "ws", optional=True), ws.numel() * ws.element_size(), _stream(stream)),
           "etp_neighbor_count")


def etp_neighbor_fill(pos, box, cutoff: float, row_ptr, n_edges: int, src, vec, ws, flags: int = 0,
                      stream=None):
    """src[E] (ascending within each row) and vec[E, 3] (minimum image of pos[src] - pos[dst])."""
    import torch
    n = pos.shape[0]
    bx = _box3(box)
    _check(lib.etp_neighbor_fill(n, _ptr(pos, "pos", torch.float32, 3 * n, optional=True), bx.ctypes.data,
                                 float(cutoff), _ptr(row_ptr, "row_ptr", torch.int32, n + 1), n_edges,
                                 _ptr(src, "src", torch.int32, n_edges, optional=True),
                                 _ptr(vec, "vec", torch.float32, 3 * n_edges, optional=True), flags,
                                 _ptr(ws, "ws", optional=True), ws.numel() * ws.element_size(), _stream(stream)),
           "etp_neighbor_fill")


def neighbor_list(pos, box, cutoff: float, flags: int = 0, stream=None):
    """Both calls with torch-allocated outputs: (row_ptr, src, vec) on pos's device.
    Reads the edge count back to the host in between (synchronises the stream)."""
    import torch
    n = pos.shape[0]
    dev = pos.device
    ws = torch.empty(etp_neighbor_workspace(n, box, cutoff), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
    etp_neighbor_count(pos, box, cutoff, row_ptr, ws, stream)
    E = int(row_ptr[n].item())
    src = torch.empty(E, dtype=torch.int32, device=dev)
    vec = torch.empty(E, 3, dtype=torch.float32, device=dev)
    etp_neighbor_fill(pos, box, cutoff, row_ptr, E, src, vec, ws, flags, stream)
    return row_ptr, src, vec
