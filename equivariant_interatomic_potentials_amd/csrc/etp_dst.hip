// etp_dst.hip -- destination-segmented passes of the edge tensor-product
// convolution: the forward, and the dG term of the VJP-of-VJP.
//
//   fwd  out[i, p, m3, u] = sum_{e in in(i)} sum_{m1} T[e, p, m1, m3] w[e, p, u] x[src_e, m1, u]
//   dG   dG[i, p, m3, u]  = sum_{e in in(i)} sum_{m1} T (w X' + W' x) + Td w x
//        with T[e, p, m1, m3] = sum_m2 C Y_m2(r_e) and Td the same with
//        Yd = grad Y . R'_e (the JVP of the forward along (X', W', R')).
//
// (the CG tensor product with sparse Wigner 3-j coefficients of "High-
// performance training and inference for deep equivariant interatomic
// potentials", section "Proposed method"; the edge-convolution forward and
// VJP-of-VJP stages of "How does FlashCart make equivariant interatomic
// potentials faster and more accurate?", section "Generated kernels beat SH
// baselines at high order").
//
// Mapping (gfx950, wave64):
//   * one workgroup per (destination node, 64*CPL-channel chunk, path
//     group); its S waves split the node's in-edges into contiguous parts; a
//     lane owns CPL consecutive channels, so every feature / weight row
//     access is one coalesced 256*CPL-byte wave load;
//   * path groups bound the per-lane register accumulators (output rows of
//     the group x CPL);
//   * per batch of B edges, lane k evaluates the SH of edge k in registers
//     and the edge-uniform T (and Td) of the group's (p, m1, m3) pairs into
//     the wave's LDS slice; the edge loop reads them as broadcast float4;
//   * messages live in registers only; the sum over a wave's edges is a
//     fixed-order register sum and the S waves meet in a fixed-order LDS
//     tree, so results are deterministic without atomics;
//   * w / W' are streamed with non-temporal loads, x / X' rows gathered
//     cached; each path's w row (and each l1 block's x rows) is reloaded
//     with the next edge's as soon as its last use in the current edge is
//     done, one edge of look-ahead in one register set;
//   * radial modes (forward, and the dG term of the radial VJP-of-VJP):
//     instead of a w stream, each path's weight is formed in registers as
//     w[e, p, u] = sum_k h[e, k] Wr[k, p, u] (the last layer of a radial
//     network) at the path's first use, and for dG also W' = sum_k H'[e, k]
//     Wr[k, p, u] from the cotangent H' on grad_h: the lane's Wr entries of
//     the group's paths stay in registers for the whole workgroup, and the
//     edge's h (and H') row is written to LDS with its SH and read back once
//     per edge (a broadcast).
#include "etp_conv_common.hpp"

namespace etp {

// Launch shape of the destination pass: S waves per workgroup, B edges per
// SH/T batch, MAXROWS output rows per path group (register accumulators =
// MAXROWS x channels per lane). The ETP_DST_* macros override the defaults
// for tuning builds.
#ifndef ETP_DST_S
#define ETP_DST_S 4
#endif
#ifndef ETP_DST_B2
#define ETP_DST_B2 32
#endif
#ifndef ETP_DST_B3
#define ETP_DST_B3 16
#endif
#ifndef ETP_DST_B4
#define ETP_DST_B4 8
#endif
#ifndef ETP_DST_ROWS_FWD
#define ETP_DST_ROWS_FWD 112
#endif
#ifndef ETP_DST_ROWS_DG
#define ETP_DST_ROWS_DG 64  // two groups at l = 2, C = 128 (40: three, 15% slower)
#endif
#ifndef ETP_DST_ROWS_FWD3
#define ETP_DST_ROWS_FWD3 ETP_DST_ROWS_FWD
#endif
#ifndef ETP_DST_ROWS_FWD3_BF16
#define ETP_DST_ROWS_FWD3_BF16 88  // bf16 features, two channels per lane (112 spills there)
#endif
#ifndef ETP_DST_ROWS_FWD4
#define ETP_DST_ROWS_FWD4 80
#endif
#ifndef ETP_DST_ROWS_DG3
#define ETP_DST_ROWS_DG3 56
#endif
#ifndef ETP_DST_ROWS_DG1
#define ETP_DST_ROWS_DG1 40
#endif
#ifndef ETP_DST_ROWS_DG4
#define ETP_DST_ROWS_DG4 24
#endif
#ifndef ETP_DST_ROWS_RAD
#define ETP_DST_ROWS_RAD 40  // radial mode at l >= 3: a group's Wr entries live in registers
#endif
#ifndef ETP_DST_WPE
#define ETP_DST_WPE 0
#endif
template <int L, int CPL, int MODE, bool BF>
struct DstCfg {
    static constexpr int S = ETP_DST_S;
    static constexpr int B = L <= 2 ? ETP_DST_B2 : (L == 3 ? ETP_DST_B3 : ETP_DST_B4);
    static constexpr int ROWS3 = (BF && CPL == 2) ? ETP_DST_ROWS_FWD3_BF16 : ETP_DST_ROWS_FWD3;
    static constexpr int ROWS = MODE == DST_DG_RADIAL ? ETP_DST_ROWS_RAD
                              : MODE == DST_FWD_RADIAL ? (L <= 2 ? ETP_DST_ROWS_FWD : ETP_DST_ROWS_RAD)
                              : MODE == DST_FWD ? (L <= 2 ? ETP_DST_ROWS_FWD : L == 3 ? ROWS3 : ETP_DST_ROWS_FWD4)
                                                : (L <= 2 ? ETP_DST_ROWS_DG : L == 3 ? ETP_DST_ROWS_DG3 : ETP_DST_ROWS_DG4);
    // (the dG pass with one channel per lane keeps 40-row groups at l <= 3:
    // one 51-row group at l = 2, C = 64 is 19% slower than two)
    static constexpr int MAXROWS =
        (MODE == DST_DG && CPL == 1 && L <= 3) ? ETP_DST_ROWS_DG1 : (ROWS + CPL - 1) / CPL;
    static constexpr int TCOPIES = (MODE == DST_DG || MODE == DST_DG_RADIAL) ? 2 : 1;  // T (and Td) per edge
    static constexpr int HROWS = MODE == DST_DG_RADIAL ? 2 : MODE == DST_FWD_RADIAL ? 1 : 0;  // h (, H') per edge
    // waves per SIMD the registers must allow: 3 at l=3 (169 VGPRs otherwise);
    // 2 in the radial mode, whose Wr entries take 8 registers per path
    static constexpr int WPE = ETP_DST_WPE > 0 ? ETP_DST_WPE
                             : (MODE == DST_FWD_RADIAL || MODE == DST_DG_RADIAL) ? 2 : (L == 3 ? 3 : 1);
};

template <int L, int CPL, typename XT, int MODE, int G>
__device__ __forceinline__ void dst_group(const int n_dst, const int C, const int nchunk,
                                          const int *__restrict__ row_ptr, const int *__restrict__ src,
                                          const float *__restrict__ vec, const XT *__restrict__ x,
                                          const float *__restrict__ w, const float *__restrict__ ggx,
                                          const float *__restrict__ ggw, const float *__restrict__ ggvec,
                                          float *__restrict__ out, const uint32_t flags, float *lds,
                                          const float *__restrict__ hrad, const float *__restrict__ wrad,
                                          const int nbasis, const float *__restrict__ ggh)
{
    using V = chv_t<CPL>;
    using Cfg = DstCfg<L, CPL, MODE, sizeof(XT) == 2>;
    constexpr int S = Cfg::S, B = Cfg::B, TC = Cfg::TCOPIES;
    constexpr bool DG = MODE == DST_DG || MODE == DST_DG_RADIAL;
    constexpr bool RAD = MODE == DST_FWD_RADIAL || MODE == DST_DG_RADIAL;
    constexpr int HROWS = Cfg::HROWS;
    constexpr int RK = kRadialMax;
    constexpr Groups GR = make_groups(kTab<L>, Cfg::MAXROWS);
    constexpr GroupInfo GI = group_info(kTab<L>, GR, G);
    constexpr int P = kTab<L>.P, DIN = kTab<L>.din_rows, DOUT = kTab<L>.dout_rows, DSH = kTab<L>.dsh;
    constexpr int NP = GI.np, NXR = GI.nxr, NROW = GI.nrow, STRIDE = GI.stride;
    constexpr int LDS_FLOATS = S * TC * B * max_stride(kTab<L>, GR);

    const int lane = threadIdx.x & 63, wv = wave_id();
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int node = lb / nchunk, chunk = lb - node * nchunk;
    if (node >= n_dst)
        return;
    const int u0 = chunk * 64 * CPL + lane * CPL;
    const bool active = u0 < C;
    // byte offsets of this lane's channels; lanes past C use an offset
    // beyond every block, so their buffer loads read 0 and stores are dropped
    const uint32_t off4 = active ? static_cast<uint32_t>(u0) * 4u : kOOB;
    const uint32_t offx = active ? static_cast<uint32_t>(u0) * static_cast<uint32_t>(sizeof(XT)) : kOOB;
    const uint32_t rowb = static_cast<uint32_t>(C) * 4u, rowx = static_cast<uint32_t>(C) * sizeof(XT);
    const bool has_xp = DG && ggx != nullptr, has_rp = DG && ggvec != nullptr;
    // W' comes from memory, or in the radial mode from the edge's H' row
    const bool has_wp = DG && (RAD ? ggh != nullptr : ggw != nullptr);

    const int rb = row_ptr[node], re = row_ptr[node + 1];
    const int len = re - rb;
    const int e_begin = rb + static_cast<int>((static_cast<int64_t>(len) * wv) / S);
    const int e_end = rb + static_cast<int>((static_cast<int64_t>(len) * (wv + 1)) / S);
    float *tl = lds + wv * (TC * B * STRIDE);  // T[B][STRIDE] (then Td[B][STRIDE])
    // radial modes: after the T slices, per wave the batch's h (and H') rows
    // [B][HROWS * RK] (zero past nbasis); the lane's Wr[k, p, u] of the
    // group's paths in registers (zero past nbasis and C)
    float *hl = lds + S * TC * B * max_stride(kTab<L>, GR) + wv * (B * HROWS * RK);
    float wr[RAD ? NP : 1][RK];
    if constexpr (RAD) {
        static_assert(CPL == 1, "the radial mode keeps one channel per lane");
        static_range<0, NP>([&](auto q) {
            static_range<0, RK>([&](auto k) {
                wr[q][k] = (active && k < nbasis) ? wrad[(static_cast<int64_t>(k) * P + GI.p0 + q) * C + u0] : 0.f;
            });
        });
    }

    V acc[NROW];
    static_range<0, NROW>([&](auto r) { acc[r] = vzero<V>(); });

    // Per-edge operands: w (and W') rows of the group's paths, x (and X')
    // rows of the group's l1 values. One register set: a path's w row is
    // reloaded with the next edge's as soon as the path is done, an l1
    // block's x rows as soon as the last path with that l1 is done (paths
    // are in l1-major order), which gives one edge of look-ahead.
    struct Ops {
        V w[NP], x[NXR], wp[DG ? NP : 1], xp[DG ? NXR : 1];
    };
    struct EdgeRsrc {
        rsrc_t w, x, wp, xp;
    };
    auto edge_rsrc = [&](int e, bool valid) {
        const int j = src[e];
        EdgeRsrc r;
        r.w = make_rsrc(RAD ? nullptr : w + static_cast<int64_t>(e) * (P * C), (!RAD && valid) ? P * C * 4u : 0u);
        r.x = make_rsrc(x + static_cast<int64_t>(j) * (DIN * C), valid ? DIN * C * static_cast<uint32_t>(sizeof(XT)) : 0u);
        // a missing cotangent is a zero-length block: its loads read 0
        r.wp = make_rsrc((has_wp && !RAD) ? ggw + static_cast<int64_t>(e) * (P * C) : nullptr,
                         (has_wp && !RAD && valid) ? P * C * 4u : 0u);
        r.xp = make_rsrc(has_xp ? ggx + static_cast<int64_t>(j) * (DIN * C) : nullptr, has_xp && valid ? DIN * C * 4u : 0u);
        return r;
    };
    Ops o;
    auto load_w = [&](auto q, const EdgeRsrc &r) {  // q: path index within the group
        if constexpr (!RAD)  // (the radial mode forms w at the path's first use)
            o.w[q] = bload<V, kNT>(r.w, off4, (GI.p0 + q) * rowb);
        if constexpr (DG && !RAD)
            o.wp[q] = bload<V, kNT>(r.wp, off4, (GI.p0 + q) * rowb);
    };
    auto load_x = [&](auto q, const EdgeRsrc &r) {  // q: x row within the group
        o.x[q] = bload_x<V, XT>(r.x, offx, (GI.xr0 + q) * rowx);
        if constexpr (DG)
            o.xp[q] = bload<V>(r.xp, off4, (GI.xr0 + q) * rowb);
    };
    auto load_all = [&](const EdgeRsrc &r) {
        static_range<0, NP>([&](auto q) { load_w(q, r); });
        static_range<0, NXR>([&](auto q) { load_x(q, r); });
    };

    // SH (and Yd) and the T (and Td) coefficients of edges [eb, eb + nb)
    auto prologue = [&](int eb, int nb) {
        wave_sync_lds();
        if (lane < nb) {
            const int e = eb + lane;
            const float rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
            if constexpr (!DG) {
                float Y[DSH];
                sh_value<L>(rx, ry, rz, Y);
                write_T<L, GI.pr0, GI.npr, STRIDE>(Y, tl + lane * STRIDE);
                if constexpr (RAD)
                    static_range<0, RK>([&](auto k) {
                        hl[lane * RK + k] = k < nbasis ? hrad[static_cast<int64_t>(e) * nbasis + k] : 0.f;
                    });
            } else {
                float px = 0.f, py = 0.f, pz = 0.f;
                if (has_rp) {
                    px = ggvec[3 * e];
                    py = ggvec[3 * e + 1];
                    pz = ggvec[3 * e + 2];
                }
                float Y[DSH], Yd[DSH];
                sh_grad_emit<L>(rx, ry, rz, [&](auto b, const D3 &y) {
                    Y[b] = y.v;
                    Yd[b] = y.g0 * px + y.g1 * py + y.g2 * pz;
                });
                write_T<L, GI.pr0, GI.npr, STRIDE>(Y, tl + lane * STRIDE);
                write_T<L, GI.pr0, GI.npr, STRIDE>(Yd, tl + B * STRIDE + lane * STRIDE);
                if constexpr (RAD)
                    static_range<0, RK>([&](auto k) {
                        hl[lane * (2 * RK) + k] = k < nbasis ? hrad[static_cast<int64_t>(e) * nbasis + k] : 0.f;
                        hl[lane * (2 * RK) + RK + k] =
                            (has_wp && k < nbasis) ? ggh[static_cast<int64_t>(e) * nbasis + k] : 0.f;
                    });
            }
        }
        wave_sync_lds();
    };

    // Forward, per pair (p, m1, m3): either acc[p, m3] += T (w x[m1]) with the
    // inputs pre-scaled by w, or y[m3] += T x[m1] followed by
    // acc[p, m3] += w y[m3], whichever form needs fewer multiplies.
    // dG: acc[p, m3] += T (w X' + W' x)[m1] + Td (w x)[m1].
    auto compute = [&](const float *tk, const float *hk, const EdgeRsrc &nx) {
        float4 tq = make_float4(0.f, 0.f, 0.f, 0.f), tdq = tq;
        V xw[9], y[9], xx[DG ? 9 : 1];
        float4 h0, h1, hp0, hp1;
        if constexpr (RAD) {
            h0 = *reinterpret_cast<const float4 *>(hk);
            h1 = *reinterpret_cast<const float4 *>(hk + 4);
            if constexpr (DG) {
                hp0 = *reinterpret_cast<const float4 *>(hk + RK);
                hp1 = *reinterpret_cast<const float4 *>(hk + RK + 4);
            }
        }
        static_range<GI.pr0, GI.pr1>([&](auto q) {
            constexpr Pair pr = kTab<L>.pair[q];
            constexpr Path pa = kTab<L>.path[pr.path];
            constexpr int d1 = 2 * pa.l1 + 1, d3 = 2 * pa.l3 + 1;
            constexpr int XO = pa.x_row - GI.xr0, OO = pa.out_row - GI.row0, WQ = pr.path - GI.p0;
            constexpr bool XW = DG || d1 <= d3;
            constexpr int a = pr.m1 + pa.l1, c3 = pr.m3 + pa.l3, ql = q - GI.pr0;
            if constexpr (RAD && q == pa.pr0) {  // w[e, p, u] = sum_k h[e, k] Wr[k, p, u], k in order
                float t = h0.x * wr[WQ][0];
                t = fmaf(h0.y, wr[WQ][1], t);
                t = fmaf(h0.z, wr[WQ][2], t);
                t = fmaf(h0.w, wr[WQ][3], t);
                t = fmaf(h1.x, wr[WQ][4], t);
                t = fmaf(h1.y, wr[WQ][5], t);
                t = fmaf(h1.z, wr[WQ][6], t);
                o.w[WQ] = fmaf(h1.w, wr[WQ][7], t);
                if constexpr (DG) {  // W'[e, p, u] = sum_k H'[e, k] Wr[k, p, u], k in order
                    float v = hp0.x * wr[WQ][0];
                    v = fmaf(hp0.y, wr[WQ][1], v);
                    v = fmaf(hp0.z, wr[WQ][2], v);
                    v = fmaf(hp0.w, wr[WQ][3], v);
                    v = fmaf(hp1.x, wr[WQ][4], v);
                    v = fmaf(hp1.y, wr[WQ][5], v);
                    v = fmaf(hp1.z, wr[WQ][6], v);
                    o.wp[WQ] = fmaf(hp1.w, wr[WQ][7], v);
                }
            }
            if constexpr (XW && q == pa.pr0) {
                static_range<0, d1>([&](auto k) {
                    xw[k] = o.w[WQ] * o.x[XO + k];
                    if constexpr (DG)
                        xx[k] = vfma(o.w[WQ], o.xp[XO + k], o.wp[WQ] * o.x[XO + k]);
                });
            }
            if constexpr (ql % 4 == 0) {
                tq = *reinterpret_cast<const float4 *>(tk + ql);
                if constexpr (DG)
                    tdq = *reinterpret_cast<const float4 *>(tk + B * STRIDE + ql);
            }
            const float t = pick4<ql % 4>(tq);
            if constexpr (DG) {
                const float td = pick4<ql % 4>(tdq);
                acc[OO + c3] = vfma(t, xx[a], vfma(td, xw[a], acc[OO + c3]));
            } else if constexpr (XW) {
                acc[OO + c3] = vfma(t, xw[a], acc[OO + c3]);
            } else if constexpr (first_m3_in_path(kTab<L>, q)) {
                y[c3] = t * o.x[XO + a];
            } else {
                y[c3] = vfma(t, o.x[XO + a], y[c3]);
            }
            if constexpr (!XW && q == pa.pr1 - 1)
                static_range<0, d3>([&](auto m) { acc[OO + m] = vfma(o.w[WQ], y[m], acc[OO + m]); });
            if constexpr (q == pa.pr1 - 1) {
                // the path is done: its w row, and the x rows of its l1 when no
                // later path of the group uses them, take the next edge's
                load_w(ic<WQ>{}, nx);
                if constexpr (pr.path + 1 == GI.p1 || kTab<L>.path[pr.path + 1].l1 != pa.l1)
                    static_range<0, d1>([&](auto k) { load_x(ic<XO + k>{}, nx); });
            }
        });
    };

    // Edges in batches of B: the batch's SH / T are evaluated first, then
    // its edges run with one edge of look-ahead. The look-ahead stops at the
    // batch end, so no operand registers are live while the next batch's SH
    // are evaluated.
    int kb = 0, nb = 0;
    for (int e = e_begin; e < e_end; ++e) {
        if (kb == 0) {
            nb = min(B, e_end - e);
            prologue(e, nb);
            load_all(edge_rsrc(e, true));
        }
        const bool more = kb + 1 < nb;
        compute(tl + kb * STRIDE, hl + kb * (HROWS * RK), edge_rsrc(more ? e + 1 : e, more));
        kb = (kb + 1 == nb) ? 0 : kb + 1;
    }

    reduce_waves<S, NROW, V, LDS_FLOATS>(acc, lds, lane, wv);

    if (wv == 0) {
        const rsrc_t ro = make_rsrc(out + static_cast<int64_t>(node) * (DOUT * C), DOUT * C * 4u);
        if (flags & 1u) {
            static_range<0, NROW>([&](auto r) {
                const uint32_t so = (GI.row0 + r) * rowb;
                bstore<V>(acc[r] + bload<V>(ro, off4, so), ro, off4, so);
            });
        } else {
            static_range<0, NROW>([&](auto r) { bstore<V>(acc[r], ro, off4, (GI.row0 + r) * rowb); });
        }
    }
}

template <int L, int CPL, typename XT, int MODE>
__global__ void __launch_bounds__((64 * DstCfg<L, CPL, MODE, sizeof(XT) == 2>::S))
    __attribute__((amdgpu_waves_per_eu(DstCfg<L, CPL, MODE, sizeof(XT) == 2>::WPE)))
    dst_kernel(const int n_dst, const int C, const int nchunk, const int *__restrict__ row_ptr,
               const int *__restrict__ src, const float *__restrict__ vec, const XT *__restrict__ x,
               const float *__restrict__ w, const float *__restrict__ ggx, const float *__restrict__ ggw,
               const float *__restrict__ ggvec, float *__restrict__ out, const uint32_t flags,
               const float *__restrict__ hrad, const float *__restrict__ wrad, const int nbasis,
               const float *__restrict__ ggh)
{
    extern __shared__ float lds[];
    constexpr Groups GR = make_groups(kTab<L>, DstCfg<L, CPL, MODE, sizeof(XT) == 2>::MAXROWS);
    const int g = blockIdx.y;
    static_range<0, GR.n>([&](auto G) __attribute__((always_inline)) {
        if (g == G)
            dst_group<L, CPL, XT, MODE, G>(n_dst, C, nchunk, row_ptr, src, vec, x, w, ggx, ggw, ggvec, out, flags,
                                           lds, hrad, wrad, nbasis, ggh);
    });
}

template <int L, int CPL, typename XT, int MODE>
static hipError_t launch_dst_t(const ConvArgs &a)
{
    using Cfg = DstCfg<L, CPL, MODE, sizeof(XT) == 2>;
    constexpr Groups GR = make_groups(kTab<L>, Cfg::MAXROWS);
    constexpr int LDS_FLOATS = Cfg::S * Cfg::TCOPIES * Cfg::B * max_stride(kTab<L>, GR) +
                               Cfg::S * Cfg::B * Cfg::HROWS * kRadialMax;
    const int nchunk = (a.C + 64 * CPL - 1) / (64 * CPL);
    const int64_t nblk = static_cast<int64_t>(a.n_dst) * nchunk;
    if (nblk == 0)
        return hipSuccess;
    if (nblk > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    dim3 grid(static_cast<unsigned>(nblk), GR.n), block(64 * Cfg::S);
    hipLaunchKernelGGL((dst_kernel<L, CPL, XT, MODE>), grid, block, LDS_FLOATS * sizeof(float), a.stream, a.n_dst,
                       a.C, nchunk, a.row_ptr, a.src, a.vec, static_cast<const XT *>(a.x), a.w, a.ggx, a.ggw,
                       a.ggvec, a.out, a.flags, a.h, a.wr, a.nbasis, a.ggh);
    return hipGetLastError();
}

#if !defined(ETP_L) || !defined(ETP_XT) || !defined(ETP_MODE)
#error "compile this file once per (l_max, dtype, mode) with -DETP_L=0..4 -DETP_XT=0|1 -DETP_MODE=0..3"
#endif

hipError_t ETP_RUN_NAME(dst, ETP_L, ETP_XT, ETP_MODE)(const ConvArgs &a)
{
    using XT = std::conditional_t<ETP_XT == 1, bf16raw, float>;
    // two channels per lane above 64 channels, except for the l_max = 4 dG
    // pass whose doubled operands (w, W', x, X') need one channel per lane
#ifndef ETP_DST_CPL1
#define ETP_DST_CPL1 0
#endif
    // (and the radial mode: its Wr slice in LDS doubles with the channels)
    constexpr bool ONE = (ETP_MODE == DST_DG && ETP_L >= 4) || ETP_MODE == DST_FWD_RADIAL || ETP_MODE == DST_DG_RADIAL ||
                         ETP_DST_CPL1;
    if constexpr (ONE)
        return launch_dst_t<ETP_L, 1, XT, ETP_MODE>(a);
    else
        return a.C > 64 ? launch_dst_t<ETP_L, 2, XT, ETP_MODE>(a) : launch_dst_t<ETP_L, 1, XT, ETP_MODE>(a);
}

}  // namespace etp
