"""Float64 CPU oracle for the fused edge tensor-product convolution.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. The product (the HIP
library and its Python binding) never imports it, and the two share no code.

This module is a thin ctypes wrapper over ``etp_oracle.c`` (plain C, double
precision, loops edge by edge). It compiles that file with gcc on first use if
the shared library is missing or older than the source.

Array conventions (all numpy, C-contiguous):
  row_ptr[n_dst+1], src[E]          int32, destination-sorted CSR
  vec[E, 3]                         bond vectors r_src - r_dst
  x[n_src, Din, C]                  Din = (lin+1)^2, row l*l + l + m
  w[E, P, C]                        per-edge, per-path, per-channel weight
  out / G[n_dst, Dout, C]           Dout = sum_p (2 l3_p + 1)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "etp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_i8p = ctypes.POINTER(ctypes.c_int8)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile etp_oracle.c into liboracle.so (gcc, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # ORACLE_LIB lets the mutation test load a deliberately broken copy
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = build()
        lib = ctypes.CDLL(path)
        lib.oracle_cg_complex.restype = ctypes.c_double
        lib.oracle_cg_complex.argtypes = [ctypes.c_int] * 6
        lib.oracle_cg_real_dense.restype = ctypes.c_double
        lib.oracle_cg_real_dense.argtypes = [ctypes.c_int] * 3 + [_f64p]
        lib.oracle_paths.restype = ctypes.c_int
        lib.oracle_paths.argtypes = [ctypes.c_int] * 3 + [_i32p, ctypes.c_int]
        lib.oracle_cg_sparse.restype = ctypes.c_int
        lib.oracle_cg_sparse.argtypes = [ctypes.c_int] * 3 + [_i32p, _i8p, _f64p, ctypes.c_int]
        lib.oracle_dims.restype = ctypes.c_int
        lib.oracle_dims.argtypes = [ctypes.c_int] * 3 + [_i32p]
        lib.oracle_sh_point.restype = None
        lib.oracle_sh_point.argtypes = [ctypes.c_int, _f64p, _f64p, _f64p, _f64p, _f64p]
        lib.oracle_sh.restype = None
        lib.oracle_sh.argtypes = [ctypes.c_int, ctypes.c_int64, _f64p, _f64p, _f64p]
        lib.oracle_transpose.restype = None
        lib.oracle_transpose.argtypes = [ctypes.c_int, ctypes.c_int, _i32p, _i32p,
                                         _i32p, _i32p, _i32p]
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_fwd.argtypes = [ctypes.c_int] * 5 + [_i32p, _i32p] + [_f64p] * 4
        lib.oracle_vjp.restype = ctypes.c_int
        lib.oracle_vjp.argtypes = [ctypes.c_int] * 6 + [_i32p, _i32p] + [_f64p] * 7
        lib.oracle_vjp2.restype = ctypes.c_int
        lib.oracle_vjp2.argtypes = [ctypes.c_int] * 6 + [_i32p, _i32p] + [_f64p] * 11
        lib.oracle_channel_mix.restype = ctypes.c_int
        lib.oracle_channel_mix.argtypes = [ctypes.c_int] * 5 + [_f64p] * 3
        lib.oracle_edge_forces.restype = None
        lib.oracle_edge_forces.argtypes = [ctypes.c_int, ctypes.c_int, _i32p, _i32p, _f64p, _f64p]
        _f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_neighbors.restype = ctypes.c_int64
        lib.oracle_neighbors.argtypes = [ctypes.c_int, _f32p, _f32p, ctypes.c_float, _i32p, _i32p, _f32p]
        lib.oracle_neighbor_row.restype = ctypes.c_int
        lib.oracle_neighbor_row.argtypes = [ctypes.c_int, _f32p, _f32p, ctypes.c_float, ctypes.c_int, _i32p, _f32p]
        lib.oracle_node_product.restype = ctypes.c_int
        lib.oracle_node_product.argtypes = [ctypes.c_int] * 4 + [_f64p, _f64p, _f64p]
        lib.oracle_node_product_vjp.restype = ctypes.c_int
        lib.oracle_node_product_vjp.argtypes = [ctypes.c_int] * 4 + [_f64p, _f64p, _f64p, _f64p]
        lib.oracle_channel_mix_vjp.restype = ctypes.c_int
        lib.oracle_channel_mix_vjp.argtypes = [ctypes.c_int] * 5 + [_f64p, _f64p, _f64p]
        lib.oracle_node_product_wgrad.restype = ctypes.c_int
        lib.oracle_node_product_wgrad.argtypes = [ctypes.c_int] * 4 + [_f64p, _f64p, _f64p, _f64p]
        lib.oracle_channel_mix_wgrad.restype = ctypes.c_int
        lib.oracle_channel_mix_wgrad.argtypes = [ctypes.c_int] * 5 + [_f64p, _f64p, _f64p]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def _lmax(L):
    if isinstance(L, (tuple, list)):
        return int(L[0]), int(L[1]), int(L[2])
    return int(L), int(L), int(L)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a, t):
    if a is None:
        return None
    return a.ctypes.data_as(t)


def num_threads() -> int:
    return _load().oracle_num_threads()


def cg_complex(j1, m1, j2, m2, J, M) -> float:
    return _load().oracle_cg_complex(j1, m1, j2, m2, J, M)


def cg_real_dense(l1, l2, l3):
    """Dense real coupling tensor [2l1+1, 2l2+1, 2l3+1] and the largest discarded part."""
    out = np.zeros((2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1), np.float64)
    disc = _load().oracle_cg_real_dense(l1, l2, l3, _p(out, _f64p))
    return out.reshape(2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1), disc


def paths(L) -> np.ndarray:
    lin, lsh, lout = _lmax(L)
    n = _load().oracle_paths(lin, lsh, lout, None, 0)
    out = np.zeros((n, 3), np.int32)
    _load().oracle_paths(lin, lsh, lout, _p(out, _i32p), n)
    return out


def cg_sparse(L):
    """(ptr[P+1], m[nnz, 3] signed m values, val[nnz]) for all paths of L."""
    lin, lsh, lout = _lmax(L)
    lib = _load()
    P = lib.oracle_paths(lin, lsh, lout, None, 0)
    nnz = lib.oracle_cg_sparse(lin, lsh, lout, None, None, None, 0)
    ptr = np.zeros(P + 1, np.int32)
    m = np.zeros((nnz, 3), np.int8)
    val = np.zeros(nnz, np.float64)
    lib.oracle_cg_sparse(lin, lsh, lout, _p(ptr, _i32p), _p(m, _i8p), _p(val, _f64p), nnz)
    return ptr, m, val


def dims(L):
    """dict(P, nnz, Din, Dsh, Dout) -- Din/Dout per channel."""
    lin, lsh, lout = _lmax(L)
    d = np.zeros(5, np.int32)
    if _load().oracle_dims(lin, lsh, lout, _p(d, _i32p)):
        raise ValueError("unsupported l_max")
    return dict(P=int(d[0]), nnz=int(d[1]), Din=int(d[2]), Dsh=int(d[3]), Dout=int(d[4]))


def sh_point(L: int, r, v=None):
    """(Y[D], dY[3, D], HV[3, D] or None) at one point r; HV_k = d/dr_k (grad Y . v)."""
    D = (L + 1) ** 2
    r = _f64(r)
    Y = np.zeros(D)
    dY = np.zeros((3, D))
    HV = np.zeros((3, D)) if v is not None else None
    vv = _f64(v) if v is not None else None
    _load().oracle_sh_point(L, _p(r, _f64p), _p(vv, _f64p), _p(Y, _f64p), _p(dY, _f64p),
                            _p(HV, _f64p))
    return Y, dY, HV


def sh(L: int, vec, grad: bool = False):
    """Y[E, D] (and dY[E, 3, D] if grad) for bond vectors vec[E, 3]."""
    vec = _f64(vec).reshape(-1, 3)
    E = vec.shape[0]
    D = (L + 1) ** 2
    Y = np.zeros((E, D))
    dY = np.zeros((E, 3, D)) if grad else None
    _load().oracle_sh(L, E, _p(vec, _f64p), _p(Y, _f64p), _p(dY, _f64p))
    return (Y, dY) if grad else Y


def transpose(row_ptr, src, n_src):
    """Stable CSR transpose: (src_ptr[n_src+1], perm[E], perm_dst[E]), int32."""
    row_ptr = _i32(row_ptr)
    src = _i32(src)
    n_dst = row_ptr.shape[0] - 1
    E = int(row_ptr[-1])
    sp = np.zeros(n_src + 1, np.int32)
    perm = np.zeros(max(E, 1), np.int32)
    pdst = np.zeros(max(E, 1), np.int32)
    _load().oracle_transpose(n_dst, n_src, _p(row_ptr, _i32p), _p(src, _i32p),
                             _p(sp, _i32p), _p(perm, _i32p), _p(pdst, _i32p))
    return sp, perm[:E], pdst[:E]


def _graph(row_ptr, src):
    row_ptr = _i32(row_ptr)
    src = _i32(src) if len(src) else np.zeros(1, np.int32)
    return row_ptr, src, row_ptr.shape[0] - 1


def fwd(L, row_ptr, src, vec, x, w):
    """out[n_dst, Dout, C]."""
    lin, lsh, lout = _lmax(L)
    row_ptr, src, n_dst = _graph(row_ptr, src)
    x = _f64(x)
    C = x.shape[2]
    d = dims(L)
    out = np.zeros((n_dst, d["Dout"], C))
    vec = _f64(vec).reshape(-1)
    w = _f64(w).reshape(-1)
    rc = _load().oracle_fwd(lin, lsh, lout, C, n_dst, _p(row_ptr, _i32p), _p(src, _i32p),
                            _p(_nz(vec), _f64p), _p(x, _f64p), _p(_nz(w), _f64p), _p(out, _f64p))
    if rc:
        raise ValueError("oracle_fwd failed")
    return out


def mix_rows(L) -> list:
    """Number of paths per output order l3 = 0..l_max_out: W_l has n_l * C rows."""
    lout = _lmax(L)[2]
    p = paths(L)
    return [int((p[:, 2] == l).sum()) for l in range(lout + 1)]


def channel_mix(L, out, W):
    """y[n, (l_max_out+1)^2, C] from the convolution output out[n, Dout, C] and
    W = W_0, W_1, ... back to back (W_l: [n_l * C, C] row-major)."""
    lin, lsh, lout = _lmax(L)
    out = _f64(out)
    n, _, C = out.shape
    W = _f64(W).reshape(-1)
    need = sum(mix_rows(L)) * C * C
    if W.size != need:
        raise ValueError(f"W has {W.size} values, expected {need}")
    y = np.zeros((n, (lout + 1) ** 2, C))
    if _load().oracle_channel_mix(lin, lsh, lout, C, n, _p(_nz(out.reshape(-1)), _f64p), _p(W, _f64p),
                                  _p(_nz(y.reshape(-1)), _f64p)):
        raise ValueError("oracle_channel_mix failed")
    return y


def channel_mix_vjp(L, gy, W):
    """gin[n, Dout, C]: the transposed mixing of the cotangent gy[n, (l_max_out+1)^2, C]."""
    lin, lsh, lout = _lmax(L)
    gy = _f64(gy)
    n, _, C = gy.shape
    W = _f64(W).reshape(-1)
    Dout = int(sum(2 * p[2] + 1 for p in paths(L)))
    gin = np.zeros((n, Dout, C))
    if _load().oracle_channel_mix_vjp(lin, lsh, lout, C, n, _p(_nz(gy.reshape(-1)), _f64p), _p(W, _f64p),
                                      _p(_nz(gin.reshape(-1)), _f64p)):
        raise ValueError("oracle_channel_mix_vjp failed")
    return gin


def channel_mix_wgrad(L, out, gy):
    """gW = W_0, W_1, ... back to back: the gradient of <gy, channel_mix(out, W)>
    with respect to W (the sum over nodes and components of out (x) gy per path)."""
    lin, lsh, lout = _lmax(L)
    out, gy = _f64(out), _f64(gy)
    n, _, C = out.shape
    gW = np.zeros(sum(mix_rows(L)) * C * C)
    if _load().oracle_channel_mix_wgrad(lin, lsh, lout, C, n, _p(_nz(out.reshape(-1)), _f64p),
                                        _p(_nz(gy.reshape(-1)), _f64p), _p(_nz(gW), _f64p)):
        raise ValueError("oracle_channel_mix_wgrad failed")
    return gW


def edge_forces(row_ptr, src, n_src, gr):
    """F[max(n_dst, n_src), 3] = sum over in-edges of gr - sum over out-edges of gr
    (forces when gr = dE/dvec and vec_e = pos[src_e] - pos[dst_e])."""
    row_ptr, srcv, n_dst = _graph(row_ptr, src)
    gr = _f64(gr).reshape(-1)
    F = np.zeros((max(n_dst, n_src), 3))
    _load().oracle_edge_forces(n_dst, n_src, _p(row_ptr, _i32p), _p(srcv, _i32p), _p(_nz(gr), _f64p),
                               _p(_nz(F.reshape(-1)), _f64p))
    return F


def neighbors(pos, box, rc):
    """Periodic neighbour list (row_ptr[n+1], src[E], vec[E, 3] float32): j != i with the
    float32 minimum-image distance strictly below rc, rows sorted by src."""
    f32p = ctypes.POINTER(ctypes.c_float)
    pos = np.ascontiguousarray(pos, np.float32)
    n = pos.shape[0]
    box = np.ascontiguousarray(np.broadcast_to(np.asarray(box, np.float32), (3,)))
    lib = _load()
    row_ptr = np.zeros(n + 1, np.int32)
    E = lib.oracle_neighbors(n, _p(pos, f32p), _p(box, f32p), float(rc), _p(row_ptr, _i32p), None, None)
    src = np.zeros(max(E, 1), np.int32)
    vec = np.zeros((max(E, 1), 3), np.float32)
    lib.oracle_neighbors(n, _p(pos, f32p), _p(box, f32p), float(rc), _p(row_ptr, _i32p), _p(src, _i32p),
                         _p(vec, f32p))
    return row_ptr, src[:E], vec[:E]


def radial_weights(h, Wr):
    """w[e, p, u] = sum_k h[e, k] Wr[k, p, u]: the last layer of a radial network
    (h: [E, K] per-edge radial features, Wr: [K, P, C])."""
    h = np.asarray(h, np.float64)
    Wr = np.asarray(Wr, np.float64)
    return np.einsum("ek,kpu->epu", h, Wr)


def fwd_radial(L, row_ptr, src, vec, x, h, Wr):
    """The forward with the per-edge weights formed from (h, Wr) first."""
    return fwd(L, row_ptr, src, vec, x, radial_weights(h, Wr))


def vjp_radial(L, row_ptr, src, vec, x, h, Wr, G):
    """VJP of the forward with radial weights, by the chain rule through
    w = h Wr: (gx, gh[E, K], gr, gWr[K, P, C]) with gh[e, k] = sum_{p,u}
    gw[e, p, u] Wr[k, p, u] and gWr[k, p, u] = sum_e h[e, k] gw[e, p, u]."""
    h = np.asarray(h, np.float64)
    Wr = np.asarray(Wr, np.float64)
    gx, gw, gr = vjp(L, row_ptr, src, vec, x, radial_weights(h, Wr), G)
    E = h.shape[0]
    gw = gw[:E]
    gh = np.einsum("epu,kpu->ek", gw, Wr)
    gWr = np.einsum("ek,epu->kpu", h, gw)
    return gx, gh, gr[:E], gWr


def vjp2_radial(L, row_ptr, src, vec, x, h, Wr, G, Xp=None, Hp=None, Rp=None):
    """VJP of vjp_radial's (gx, gh, gr) with cotangents (X', H', R') on them:
    S = <X', gx> + <H', gh> + <R', gr>. Since gh = gw Wr (per edge, summed
    over paths and channels), <H', gh> = <W', gw> with W'[e, p, u] =
    sum_k H'[e, k] Wr[k, p, u], so the convolution's VJP-of-VJP with (X', W',
    R') gives (dx, dw, dr, dG); then, through w = h Wr, dh[e, k] =
    sum_{p,u} dw[e, p, u] Wr[k, p, u], and dWr[k, p, u] = sum_e h[e, k]
    dw[e, p, u] + sum_e H'[e, k] gw[e, p, u] (S also depends on Wr through
    gh). Returns (dx, dh[E, K], dr, dG, dWr[K, P, C]); None cotangent = 0."""
    h = np.asarray(h, np.float64)
    Wr = np.asarray(Wr, np.float64)
    E = h.shape[0]
    w = radial_weights(h, Wr)
    Wp = radial_weights(Hp, Wr) if Hp is not None else None
    dx, dw, dr, dG = vjp2(L, row_ptr, src, vec, x, w, G, Xp, Wp, Rp)
    dw = dw[:E]
    dh = np.einsum("epu,kpu->ek", dw, Wr)
    dWr = np.einsum("ek,epu->kpu", h, dw)
    if Hp is not None:
        gw = vjp(L, row_ptr, src, vec, x, w, G)[1][:E]
        dWr = dWr + np.einsum("ek,epu->kpu", np.asarray(Hp, np.float64), gw)
    return dx, dh, dr[:E], dG, dWr


def edge_tp_fwd(L, vec, V, w):
    """Edge-local tensor product: the convolution with every edge its own
    destination and source (out[E, Dout, C], no destination sum)."""
    E = np.asarray(vec).reshape(-1, 3).shape[0]
    ar = np.arange(E + 1, dtype=np.int32)
    return fwd(L, ar, ar[:E], vec, V, w)


def edge_tp_vjp(L, vec, V, w, G):
    """(gV, gw, gr) of the edge-local tensor product."""
    E = np.asarray(vec).reshape(-1, 3).shape[0]
    ar = np.arange(E + 1, dtype=np.int32)
    return vjp(L, ar, ar[:E], vec, V, w, G)


def edge_tp_vjp2(L, vec, V, w, G, ggV=None, ggw=None, ggvec=None):
    """(dV, dw, dr, dG) of the edge-local tensor product's VJP-of-VJP."""
    E = np.asarray(vec).reshape(-1, 3).shape[0]
    ar = np.arange(E + 1, dtype=np.int32)
    return vjp2(L, ar, ar[:E], vec, V, w, G, ggV, ggw, ggvec)


def node_product(L, A, W, nu):
    """Node-local correlation product: out[n, (L+1)^2, C] = B_1 + ... + B_nu with
    B_1 = A and B_{k+1} = sum_p W[k-1, p] * CG_p(B_k, A), channel-wise."""
    A = np.ascontiguousarray(A, np.float64)
    n, D, C = A.shape
    assert D == (L + 1) ** 2
    W = np.ascontiguousarray(np.zeros((1,)) if W is None else W, np.float64)
    out = np.zeros_like(A)
    if _load().oracle_node_product(L, C, n, nu, _p(A, _f64p), _p(W, _f64p), _p(out, _f64p)):
        raise ValueError("bad arguments")
    return out


def node_product_vjp(L, A, W, G, nu):
    """gA[n, (L+1)^2, C] = d<G, node_product(L, A, W, nu)>/dA."""
    A = np.ascontiguousarray(A, np.float64)
    n, D, C = A.shape
    G = np.ascontiguousarray(G, np.float64)
    W = np.ascontiguousarray(np.zeros((1,)) if W is None else W, np.float64)
    gA = np.zeros_like(A)
    if _load().oracle_node_product_vjp(L, C, n, nu, _p(A, _f64p), _p(W, _f64p), _p(G, _f64p), _p(gA, _f64p)):
        raise ValueError("bad arguments")
    return gA


def node_product_wgrad(L, A, W, G, nu):
    """gW[nu-1, P, C] = d<G, node_product(L, A, W, nu)>/dW (a sum over nodes)."""
    A = np.ascontiguousarray(A, np.float64)
    n, D, C = A.shape
    G = np.ascontiguousarray(G, np.float64)
    P = len(paths(L))
    W = np.ascontiguousarray(np.zeros((1,)) if W is None else W, np.float64)
    gW = np.zeros((max(nu - 1, 0), P, C))
    if _load().oracle_node_product_wgrad(L, C, n, nu, _p(A, _f64p), _p(W, _f64p), _p(G, _f64p),
                                         _p(_nz(gW.reshape(-1)), _f64p)):
        raise ValueError("bad arguments")
    return gW


def neighbor_row(pos, box, rc, i):
    """Row i of the periodic neighbour list: (src ascending, vec[k, 3])."""
    f32p = ctypes.POINTER(ctypes.c_float)
    pos = np.ascontiguousarray(pos, np.float32)
    box = np.ascontiguousarray(np.broadcast_to(np.asarray(box, np.float32), (3,)))
    n = pos.shape[0]
    src = np.zeros(max(n, 1), np.int32)
    vec = np.zeros((max(n, 1), 3), np.float32)
    k = _load().oracle_neighbor_row(n, _p(pos, f32p), _p(box, f32p), float(rc), int(i), _p(src, _i32p),
                                    _p(vec, f32p))
    return src[:k], vec[:k]


def _nz(a):
    return a if a.size else np.zeros(1)


def vjp(L, row_ptr, src, vec, x, w, G):
    """(gx[n_src, Din, C], gw[E, P, C], gr[E, 3])."""
    lin, lsh, lout = _lmax(L)
    row_ptr, src, n_dst = _graph(row_ptr, src)
    x = _f64(x)
    n_src, _, C = x.shape
    E = int(row_ptr[-1])
    d = dims(L)
    gx = np.zeros_like(x)
    gw = np.zeros((max(E, 1), d["P"], C))
    gr = np.zeros((max(E, 1), 3))
    rc = _load().oracle_vjp(lin, lsh, lout, C, n_dst, n_src, _p(row_ptr, _i32p), _p(src, _i32p),
                            _p(_nz(_f64(vec).reshape(-1)), _f64p), _p(x, _f64p),
                            _p(_nz(_f64(w).reshape(-1)), _f64p), _p(_nz(_f64(G).reshape(-1)), _f64p),
                            _p(gx, _f64p), _p(gw, _f64p), _p(gr, _f64p))
    if rc:
        raise ValueError("oracle_vjp failed")
    return gx, gw[:E], gr[:E]


def vjp2(L, row_ptr, src, vec, x, w, G, Xp=None, Wp=None, Rp=None):
    """(dx[n_src, Din, C], dw[E, P, C], dr[E, 3], dG[n_dst, Dout, C]); None cotangent = 0."""
    lin, lsh, lout = _lmax(L)
    row_ptr, src, n_dst = _graph(row_ptr, src)
    x = _f64(x)
    n_src, _, C = x.shape
    E = int(row_ptr[-1])
    d = dims(L)
    dx = np.zeros_like(x)
    dw = np.zeros((max(E, 1), d["P"], C))
    dr = np.zeros((max(E, 1), 3))
    dG = np.zeros((n_dst, d["Dout"], C))
    Xp = _f64(Xp) if Xp is not None else None
    Wp = _nz(_f64(Wp).reshape(-1)) if Wp is not None else None
    Rp = _nz(_f64(Rp).reshape(-1)) if Rp is not None else None
    rc = _load().oracle_vjp2(lin, lsh, lout, C, n_dst, n_src, _p(row_ptr, _i32p), _p(src, _i32p),
                             _p(_nz(_f64(vec).reshape(-1)), _f64p), _p(x, _f64p),
                             _p(_nz(_f64(w).reshape(-1)), _f64p),
                             _p(_nz(_f64(G).reshape(-1)), _f64p),
                             _p(Xp, _f64p), _p(Wp, _f64p), _p(Rp, _f64p),
                             _p(dx, _f64p), _p(dw, _f64p), _p(dr, _f64p), _p(dG, _f64p))
    if rc:
        raise ValueError("oracle_vjp2 failed")
    return dx, dw[:E], dr[:E], dG
