// etp_src.hip -- source-segmented passes of the edge tensor-product
// convolution's backward: the VJP (forces) and the source half of the
// VJP-of-VJP (force training), the two derivative stages measured for the
// edge convolution in "How does FlashCart make equivariant interatomic
// potentials faster and more accurate?" (section "Generated kernels beat SH
// baselines at high order").
//
// For edge e = (i <- j), with K[p, m1, m2] = sum_m3 C G[i, p, m3]:
//   VJP   gx[j, m1]  += w s[m1],            s[m1] = sum_m2 Y_m2 K[m1, m2]
//         gw[e, p]    = sum_m1 x[j, m1] s[m1]
//         gr[e]       = sum_b Z_b dY_b/dr,  Z_b   = sum_{p,u,m1} w x[j, m1] K[m1, b]
//   VJP2  dx[j, m1]  += W' s[m1] + w sd[m1], sd[m1] = sum_m2 Yd_m2 K[m1, m2]
//         dw[e, p]    = sum_m1 X'[m1] s[m1] + x[m1] sd[m1]
//         dr[e]       = sum_b Z1_b dY_b/dr + Z2_b d(grad Y_b . R')/dr,
//         Z1_b = sum (w X' + W' x) K,  Z2_b = sum w x K,  Yd = grad Y . R'.
//
// Mapping (gfx950, wave64):
//   * one workgroup per source node j; its S waves split j's out-edges
//     (the stable transpose of the destination-sorted CSR) into contiguous
//     parts; a lane owns CPL = C/64 channels (C <= 128) so Z reduces within
//     one wave;
//   * x[j] (and X'[j]) rows and the gx / dx accumulators stay in registers;
//     G[i] rows are gathered per path (cached), w / W' streamed
//     non-temporally, gw / dw written once per edge;
//   * per batch of B edges, lane k evaluates the SH of edge k (and Yd) into
//     LDS; per edge the wave reads them as broadcast float4;
//   * Z is reduced over the wave with DPP in a fixed order, parked in LDS,
//     and at the end of the batch lane k turns it into gr / dr of edge k with
//     forward-mode SH derivatives; no float atomics anywhere.
#include "etp_conv_common.hpp"

namespace etp {

template <int L, int CPL>
struct SrcCfg {
    static constexpr int S = 4;
    static constexpr int B = L <= 2 ? 64 : 32;
    static constexpr int MAXCOST = 40 / CPL;
};

template <int L, int CPL, typename XT, int MODE, int SG>
__device__ __forceinline__ void src_group(const int n_src, const int C, const int *__restrict__ src_ptr,
                                          const int *__restrict__ perm, const int *__restrict__ perm_dst,
                                          const float *__restrict__ vec, const XT *__restrict__ x,
                                          const float *__restrict__ w, const float *__restrict__ G,
                                          const float *__restrict__ ggx, const float *__restrict__ ggw,
                                          const float *__restrict__ ggvec, float *__restrict__ ox,
                                          float *__restrict__ ow, float *__restrict__ ovec,
                                          const uint32_t flags, float *lds)
{
    using V = chv_t<CPL>;
    using Cfg = SrcCfg<L, CPL>;
    constexpr int S = Cfg::S, B = Cfg::B;
    constexpr Groups GR = make_src_groups(kTab<L>, Cfg::MAXCOST);
    constexpr SrcGroupInfo GI = src_group_info(kTab<L>, GR, SG);
    constexpr int P = kTab<L>.P, DIN = kTab<L>.din_rows, DOUT = kTab<L>.dout_rows, DSH = kTab<L>.dsh;
    constexpr int NXR = GI.nxr;
    constexpr int BLO = sh_lo(kTab<L>, GI.p0, GI.p1), BHI = sh_hi(kTab<L>, GI.p0, GI.p1);
    constexpr int DSHP = (DSH + 3) & ~3;
    constexpr bool V2 = MODE == SRC_VJP2;
    // per-wave LDS: Y[B][DSHP] (+ Yd[B][DSHP]) and Z[B][DSH] (+ Z2[B][DSH])
    constexpr int WAVE_FLOATS = (V2 ? 2 : 1) * B * (DSHP + DSH);

    const int lane = threadIdx.x & 63, wv = wave_id();
    const int j = xcd_remap(blockIdx.x, gridDim.x);
    if (j >= n_src)
        return;
    const int u0 = lane * CPL;
    const bool active = u0 < C;
    const bool want_vec = ovec != nullptr;
    const bool has_xp = V2 && ggx != nullptr, has_wp = V2 && ggw != nullptr, has_rp = V2 && ggvec != nullptr;

    float *ylds = lds + wv * WAVE_FLOATS;         // Y, then Yd
    float *zlds = ylds + (V2 ? 2 : 1) * B * DSHP;  // Z, then Z2

    const int kb0 = src_ptr[j], kb1 = src_ptr[j + 1];
    const int len = kb1 - kb0;
    const int k_begin = kb0 + static_cast<int>((static_cast<int64_t>(len) * wv) / S);
    const int k_end = kb0 + static_cast<int>((static_cast<int64_t>(len) * (wv + 1)) / S);

    // node-resident rows of x[j] (and X'[j]) for this group's l1 values
    V xr[NXR], xpr[NXR], acc[NXR];
    {
        const XT *xj = x + static_cast<int64_t>(j) * (DIN * C) + u0;
        const float *xpj = has_xp ? ggx + static_cast<int64_t>(j) * (DIN * C) + u0 : nullptr;
        static_range<0, NXR>([&](auto q) {
            xr[q] = active ? load_cached<V>(xj + (GI.xr0 + q) * C) : vzero<V>();
            xpr[q] = (has_xp && active) ? load_cached<V>(xpj + (GI.xr0 + q) * C) : vzero<V>();
            acc[q] = vzero<V>();
        });
    }

    auto prologue = [&](int kb, int nb) {
        wave_sync_lds();
        if (lane < nb) {
            const int e = perm[kb + lane];
            const float rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
            float *yp = ylds + lane * DSHP;
            if constexpr (!V2) {
                float Y[DSH], yv[DSHP];
                sh_value<L>(rx, ry, rz, Y);
                static_range<0, DSHP>([&](auto b) {
                    if constexpr (b < DSH)
                        yv[b] = Y[b];
                    else
                        yv[b] = 0.f;
                });
                static_range<0, DSHP / 4>([&](auto q) {
                    *reinterpret_cast<float4 *>(yp + 4 * q) =
                        make_float4(yv[4 * q], yv[4 * q + 1], yv[4 * q + 2], yv[4 * q + 3]);
                });
            } else {
                D3 Y[DSH];
                sh_grad<L>(rx, ry, rz, Y);
                float px = 0.f, py = 0.f, pz = 0.f;
                if (has_rp) {
                    px = ggvec[3 * e];
                    py = ggvec[3 * e + 1];
                    pz = ggvec[3 * e + 2];
                }
                float *ydp = ylds + B * DSHP + lane * DSHP;
                static_range<0, DSHP>([&](auto b) {
                    if constexpr (b < DSH) {
                        yp[b] = Y[b].v;
                        ydp[b] = Y[b].g0 * px + Y[b].g1 * py + Y[b].g2 * pz;
                    } else {
                        yp[b] = 0.f;
                        ydp[b] = 0.f;
                    }
                });
            }
        }
        wave_sync_lds();
    };

    // gr / dr of the batch's edges from the parked Z sums (lane = edge).
    auto epilogue = [&](int kb, int nb) {
        wave_sync_lds();
        if (want_vec && lane < nb) {
            const int e = perm[kb + lane];
            const float rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
            const float *zp = zlds + lane * DSH;
            float g0 = 0.f, g1 = 0.f, g2 = 0.f;
            if constexpr (!V2) {
                D3 Y[DSH];
                sh_grad<L>(rx, ry, rz, Y);
                static_range<BLO, BHI>([&](auto b) {
                    const float z = zp[b];
                    g0 = fmaf(z, Y[b].g0, g0);
                    g1 = fmaf(z, Y[b].g1, g1);
                    g2 = fmaf(z, Y[b].g2, g2);
                });
            } else {
                float px = 0.f, py = 0.f, pz = 0.f;
                if (has_rp) {
                    px = ggvec[3 * e];
                    py = ggvec[3 * e + 1];
                    pz = ggvec[3 * e + 2];
                }
                Jet Y[DSH];
                sh_jet<L>(rx, ry, rz, px, py, pz, Y);
                const float *z2p = zlds + B * DSH + lane * DSH;
                static_range<BLO, BHI>([&](auto b) {
                    const float z1 = zp[b], z2 = z2p[b];
                    g0 = fmaf(z1, Y[b].b0, fmaf(z2, Y[b].d0, g0));
                    g1 = fmaf(z1, Y[b].b1, fmaf(z2, Y[b].d1, g1));
                    g2 = fmaf(z1, Y[b].b2, fmaf(z2, Y[b].d2, g2));
                });
            }
            float *gp = ovec + 3 * static_cast<int64_t>(e);
            if (SG > 0) {  // later source groups add to the earlier groups' result
                g0 += gp[0];
                g1 += gp[1];
                g2 += gp[2];
            }
            gp[0] = g0;
            gp[1] = g1;
            gp[2] = g2;
        }
        wave_sync_lds();
    };

    int kb = 0;
    for (int k = k_begin; k < k_end; ++k) {
        const int batch0 = k - kb;
        const int nb = min(B, k_end - batch0);
        if (kb == 0)
            prologue(k, nb);
        const int e = perm[k], i = perm_dst[k];
        const float *wrow = w + static_cast<int64_t>(e) * (P * C) + u0;
        const float *wprow = has_wp ? ggw + static_cast<int64_t>(e) * (P * C) + u0 : nullptr;
        const float *grow = G + static_cast<int64_t>(i) * (DOUT * C) + u0;
        float *owrow = ow ? ow + static_cast<int64_t>(e) * (P * C) + u0 : nullptr;
        const float *yk = ylds + kb * DSHP;
        const float *ydk = ylds + B * DSHP + kb * DSHP;

        // broadcast SH (and Yd) of this edge
        float Yb[DSHP], Ydb[V2 ? DSHP : 1];
        static_range<0, DSHP / 4>([&](auto q) {
            const float4 v = *reinterpret_cast<const float4 *>(yk + 4 * q);
            Yb[4 * q] = v.x;
            Yb[4 * q + 1] = v.y;
            Yb[4 * q + 2] = v.z;
            Yb[4 * q + 3] = v.w;
            if constexpr (V2) {
                const float4 d = *reinterpret_cast<const float4 *>(ydk + 4 * q);
                Ydb[4 * q] = d.x;
                Ydb[4 * q + 1] = d.y;
                Ydb[4 * q + 2] = d.z;
                Ydb[4 * q + 3] = d.w;
            }
        });

        V Z[DSH], Z2[V2 ? DSH : 1];
        static_range<0, DSH>([&](auto b) {
            if constexpr (!ab_touches_b(kTab<L>, GI.ab0, GI.ab1, b)) {
                Z[b] = vzero<V>();
                if constexpr (V2)
                    Z2[b] = vzero<V>();
            }
        });

        static_range<GI.p0, GI.p1>([&](auto p) {
            constexpr Path pa = kTab<L>.path[p];
            constexpr int d1 = 2 * pa.l1 + 1, d3 = 2 * pa.l3 + 1;
            constexpr int XO = pa.x_row - GI.xr0;
            const V wp = active ? load_stream<V>(wrow + p * C) : vzero<V>();
            V wpp = vzero<V>();
            if constexpr (V2)
                wpp = (has_wp && active) ? load_stream<V>(wprow + p * C) : vzero<V>();
            V gv[d3];
            static_range<0, d3>([&](auto m) {
                gv[m] = active ? load_cached<V>(grow + (pa.out_row + m) * C) : vzero<V>();
            });
            V wx[d1], xx[V2 ? d1 : 1], s[d1], sd[V2 ? d1 : 1];
            static_range<0, d1>([&](auto a) {
                wx[a] = wp * xr[XO + a];
                if constexpr (V2)
                    xx[a] = vfma(wp, xpr[XO + a], wpp * xr[XO + a]);
            });
            static_range<kTab<L>.path_ab0[p], kTab<L>.path_ab0[p + 1]>([&](auto g) {
                constexpr ABGroup ag = kTab<L>.ab[g];
                constexpr int a = ag.m1 + pa.l1, b = pa.y_row + pa.l2 + ag.m2;
                V K;
                static_range<ag.t0, ag.t1>([&](auto ti) {
                    constexpr Entry en = kTab<L>.nz[kTab<L>.ab_entries[ti]];
                    if constexpr (ti == ag.t0)
                        K = en.fval * gv[en.m3 + pa.l3];
                    else
                        K = vfma(en.fval, gv[en.m3 + pa.l3], K);
                });
                if constexpr (ab_first_m1(kTab<L>, g)) {
                    s[a] = Yb[b] * K;
                    if constexpr (V2)
                        sd[a] = Ydb[b] * K;
                } else {
                    s[a] = vfma(Yb[b], K, s[a]);
                    if constexpr (V2)
                        sd[a] = vfma(Ydb[b], K, sd[a]);
                }
                if constexpr (!V2) {
                    if constexpr (ab_first_b(kTab<L>, GI.ab0, g))
                        Z[b] = wx[a] * K;
                    else
                        Z[b] = vfma(wx[a], K, Z[b]);
                } else {
                    if constexpr (ab_first_b(kTab<L>, GI.ab0, g)) {
                        Z[b] = xx[a] * K;
                        Z2[b] = wx[a] * K;
                    } else {
                        Z[b] = vfma(xx[a], K, Z[b]);
                        Z2[b] = vfma(wx[a], K, Z2[b]);
                    }
                }
            });
            // node accumulators and the per-edge weight cotangent
            V gwv;
            static_range<0, d1>([&](auto a) {
                if constexpr (!V2) {
                    acc[XO + a] = vfma(wp, s[a], acc[XO + a]);
                    if constexpr (a == 0)
                        gwv = xr[XO + a] * s[a];
                    else
                        gwv = vfma(xr[XO + a], s[a], gwv);
                } else {
                    acc[XO + a] = vfma(wpp, s[a], vfma(wp, sd[a], acc[XO + a]));
                    if constexpr (a == 0)
                        gwv = vfma(xpr[XO + a], s[a], xr[XO + a] * sd[a]);
                    else
                        gwv = vfma(xpr[XO + a], s[a], vfma(xr[XO + a], sd[a], gwv));
                }
            });
            if (owrow && active)
                __builtin_nontemporal_store(gwv, reinterpret_cast<V *>(owrow + p * C));
        });

        if (want_vec) {
            // channel sums, then the fixed-order DPP wave sum; lane 63 parks them
            float *zk = zlds + kb * DSH;
            static_range<BLO, BHI>([&](auto b) {
                float z;
                if constexpr (CPL == 1)
                    z = Z[b];
                else
                    z = Z[b].x + Z[b].y;
                z = wave_sum_to_lane63(z);
                if (lane == 63)
                    zk[b] = z;
                if constexpr (V2) {
                    float z2;
                    if constexpr (CPL == 1)
                        z2 = Z2[b];
                    else
                        z2 = Z2[b].x + Z2[b].y;
                    z2 = wave_sum_to_lane63(z2);
                    if (lane == 63)
                        zk[B * DSH + b] = z2;
                }
            });
        }

        ++kb;
        if (kb == nb) {
            epilogue(batch0, nb);
            kb = 0;
        }
    }

    // combine the S waves' node accumulators and store gx / dx rows of j
    constexpr int LDS_FLOATS = S * WAVE_FLOATS;
    reduce_waves<S, NXR, V, LDS_FLOATS>(acc, lds, lane, wv);
    if (ox && wv == 0 && active) {
        float *op = ox + static_cast<int64_t>(j) * (DIN * C) + u0 + GI.xr0 * C;
        if (flags & 1u) {
            static_range<0, NXR>([&](auto r) { store_v<V>(op + r * C, acc[r] + load_cached<V>(op + r * C)); });
        } else {
            static_range<0, NXR>([&](auto r) { store_v<V>(op + r * C, acc[r]); });
        }
    }
}

template <int L, int CPL, typename XT, int MODE, int SG>
__global__ void __launch_bounds__((64 * SrcCfg<L, CPL>::S))
    src_kernel(const int n_src, const int C, const int *__restrict__ src_ptr, const int *__restrict__ perm,
               const int *__restrict__ perm_dst, const float *__restrict__ vec, const XT *__restrict__ x,
               const float *__restrict__ w, const float *__restrict__ G, const float *__restrict__ ggx,
               const float *__restrict__ ggw, const float *__restrict__ ggvec, float *__restrict__ ox,
               float *__restrict__ ow, float *__restrict__ ovec, const uint32_t flags)
{
    extern __shared__ float lds[];
    src_group<L, CPL, XT, MODE, SG>(n_src, C, src_ptr, perm, perm_dst, vec, x, w, G, ggx, ggw, ggvec, ox, ow,
                                    ovec, flags, lds);
}

template <int L, int CPL, typename XT, int MODE>
static hipError_t launch_src_t(const ConvArgs &a)
{
    using Cfg = SrcCfg<L, CPL>;
    constexpr Groups GR = make_src_groups(kTab<L>, Cfg::MAXCOST);
    constexpr int DSH = kTab<L>.dsh, DSHP = (DSH + 3) & ~3;
    constexpr int WAVE_FLOATS = (MODE == SRC_VJP2 ? 2 : 1) * Cfg::B * (DSHP + DSH);
    constexpr size_t lds_bytes = sizeof(float) * Cfg::S * WAVE_FLOATS;
    if (a.n_src == 0)
        return hipSuccess;
    hipError_t err = hipSuccess;
    // one launch per source group, in order: later groups add to gr / dr
    static_range<0, GR.n>([&](auto g) {
        if (err != hipSuccess)
            return;
        hipLaunchKernelGGL((src_kernel<L, CPL, XT, MODE, g>), dim3(a.n_src), dim3(64 * Cfg::S), lds_bytes, a.stream,
                           a.n_src, a.C, a.src_ptr, a.perm, a.perm_dst, a.vec, static_cast<const XT *>(a.x), a.w,
                           a.G, a.ggx, a.ggw, a.ggvec, a.ox, a.ow, a.ovec, a.flags);
        err = hipGetLastError();
    });
    return err;
}

#if !defined(ETP_L) || !defined(ETP_XT) || !defined(ETP_MODE)
#error "compile this file once per (l_max, dtype, mode) with -DETP_L=0..4 -DETP_XT=0|1 -DETP_MODE=0|1"
#endif

hipError_t ETP_RUN_NAME(src, ETP_L, ETP_XT, ETP_MODE)(const ConvArgs &a)
{
    using XT = std::conditional_t<ETP_XT == 1, bf16raw, float>;
    return a.C > 64 ? launch_src_t<ETP_L, 2, XT, ETP_MODE>(a) : launch_src_t<ETP_L, 1, XT, ETP_MODE>(a);
}

}  // namespace etp
