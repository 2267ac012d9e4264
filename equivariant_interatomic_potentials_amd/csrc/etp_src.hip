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
//   * one workgroup per source node j with one wave per (64-channel chunk,
//     edge split): the splits divide j's out-edges (the stable transpose of
//     the destination-sorted CSR) into contiguous parts; a wave's gx / dx
//     rows stay in registers and the splits meet in a fixed-order LDS sum at
//     the end; every wave runs the same number of SH batches so workgroup
//     barriers stay aligned;
//   * x[j] (and X'[j]) rows stay in registers; per edge the wave streams the
//     w (and W') rows of its path group and gathers the group's G[i] rows
//     with raw buffer loads (lanes past C read 0 and their stores are
//     dropped by the buffer range check, so there are no branches around
//     memory operations); the next edge's operands are loaded before the
//     current edge's FMAs;
//   * per batch of B edges each wave evaluates the SH of the batch (lane =
//     edge) into its LDS slice; the edge loop reads them as broadcast float4;
//   * Z is reduced over each wave's lanes with DPP in a fixed order, parked
//     in LDS per chunk, and at the end of the batch lane k of wave 0 sums the
//     chunks in order and turns Z into gr / dr of edge k with forward-mode SH
//     derivatives; no float atomics anywhere.
#include "etp_conv_common.hpp"

namespace etp {

// Launch shape of the source pass: B edges per SH batch, MAXCOST bounds the
// registers of one path group (see make_src_groups). The ETP_SRC_* macros
// override the defaults for tuning builds.
#ifndef ETP_SRC_B2
#define ETP_SRC_B2 64
#endif
#ifndef ETP_SRC_COST2
#define ETP_SRC_COST2 60
#endif
#ifndef ETP_SRC_WPE
#define ETP_SRC_WPE 2
#endif
template <int L, int MODE>
struct SrcCfg {
    static constexpr int B = L <= 2 ? ETP_SRC_B2 : 32;
    static constexpr int WMUL = MODE == SRC_VJP2 ? 2 : 1;
    static constexpr int MAXCOST = L <= 2 ? ETP_SRC_COST2 : (L == 3 ? 32 : 40);
};

// Edge splits per channel chunk: four waves per workgroup in total.
constexpr int src_splits(int nch) { return nch >= 4 ? 1 : 4 / nch; }

template <int L, int MODE>
constexpr int src_lds_floats(int nch)
{
    constexpr int DSH = kTab<L>.dsh, DSHP = (DSH + 3) & ~3;
    constexpr int NV = MODE == SRC_VJP2 ? 2 : 1;
    const int nw = nch * src_splits(nch);
    const int batch = nw * NV * SrcCfg<L, MODE>::B * (DSHP + DSH);
    const int reduce = (src_splits(nch) - 1) * nch * kTab<L>.din_rows * 64;  // node rows of the splits
    return batch > reduce ? batch : reduce;
}

template <int L, typename XT, int MODE, int SG>
__device__ __forceinline__ void src_group(const int n_src, const int C, const int *__restrict__ src_ptr,
                                          const int *__restrict__ perm, const int *__restrict__ perm_dst,
                                          const float *__restrict__ vec, const XT *__restrict__ x,
                                          const float *__restrict__ w, const float *__restrict__ G,
                                          const float *__restrict__ ggx, const float *__restrict__ ggw,
                                          const float *__restrict__ ggvec, float *__restrict__ ox,
                                          float *__restrict__ ow, float *__restrict__ ovec,
                                          const uint32_t flags, float *lds)
{
    using Cfg = SrcCfg<L, MODE>;
    constexpr int B = Cfg::B;
    constexpr bool V2 = MODE == SRC_VJP2;
    constexpr Groups GR = make_src_groups(kTab<L>, Cfg::MAXCOST, Cfg::WMUL);
    constexpr SrcGroupInfo GI = src_group_info(kTab<L>, GR, SG);
    constexpr int P = kTab<L>.P, DIN = kTab<L>.din_rows, DOUT = kTab<L>.dout_rows, DSH = kTab<L>.dsh;
    constexpr int NP = GI.np, NXR = GI.nxr, NGR = GI.ngr;
    constexpr int BLO = sh_lo(kTab<L>, GI.p0, GI.p1), BHI = sh_hi(kTab<L>, GI.p0, GI.p1);
    constexpr int DSHP = (DSH + 3) & ~3;
    constexpr int NV = V2 ? 2 : 1;  // SH copies (Y, Yd) and Z copies (Z1, Z2)

    const int lane = threadIdx.x & 63, wv = wave_id();
    const int nch = (C + 63) >> 6, nsp = src_splits(nch);
    const int ch = wv % nch, sp = wv / nch;  // channel chunk, edge split
    const int j = xcd_remap(blockIdx.x, gridDim.x);
    if (j >= n_src)
        return;
    const int u = ch * 64 + lane;
    const bool active = u < C;
    const uint32_t off4 = active ? static_cast<uint32_t>(u) * 4u : kOOB;
    const uint32_t offx = active ? static_cast<uint32_t>(u) * static_cast<uint32_t>(sizeof(XT)) : kOOB;
    const bool want_vec = ovec != nullptr;
    const bool has_xp = V2 && ggx != nullptr, has_wp = V2 && ggw != nullptr, has_rp = V2 && ggvec != nullptr;
    const uint32_t rowb = static_cast<uint32_t>(C) * 4u;  // bytes per f32 row

    // LDS: per wave Y[B][DSHP] (+ Yd[B][DSHP]); then per wave Z[B][DSH] (+ Z2[B][DSH])
    const int nw = nch * nsp;
    float *ylds = lds + wv * (NV * B * DSHP);
    float *zall = lds + nw * (NV * B * DSHP);
    float *zlds = zall + wv * (NV * B * DSH);

    // this wave's split of j's out-edges; every wave runs nbatch batches
    const int len = src_ptr[j + 1] - src_ptr[j];
    const int part = (len + nsp - 1) / nsp;
    const int kb0 = src_ptr[j] + min(len, sp * part), kb1 = src_ptr[j] + min(len, (sp + 1) * part);
    const int nbatch = (part + B - 1) / B;

    // node-resident rows of x[j] (and X'[j]) for this group's l1 values
    float xr[NXR], xpr[NXR], acc[NXR];
    {
        const rsrc_t rx = make_rsrc(x + static_cast<int64_t>(j) * (DIN * C), DIN * C * sizeof(XT));
        const rsrc_t rxp = make_rsrc(has_xp ? ggx + static_cast<int64_t>(j) * (DIN * C) : nullptr,
                                     has_xp ? DIN * C * 4u : 0u);
        static_range<0, NXR>([&](auto q) {
            xr[q] = bload_x<float, XT>(rx, offx, (GI.xr0 + q) * C * sizeof(XT));
            xpr[q] = V2 ? bload<float>(rxp, off4, (GI.xr0 + q) * rowb) : 0.f;
            acc[q] = 0.f;
        });
    }

    struct Ops {
        float w[NP], wp[V2 ? NP : 1], g[NGR];
    };
    auto load = [&](int k, Ops &o) {
        const int e = perm[k], i = perm_dst[k];
        const rsrc_t rw = make_rsrc(w + static_cast<int64_t>(e) * (P * C), P * C * 4u);
        const rsrc_t rg = make_rsrc(G + static_cast<int64_t>(i) * (DOUT * C), DOUT * C * 4u);
        static_range<0, NP>([&](auto q) { o.w[q] = bload<float, kNT>(rw, off4, (GI.p0 + q) * rowb); });
        static_range<0, NGR>([&](auto r) { o.g[r] = bload<float>(rg, off4, (GI.gr0 + r) * rowb); });
        if constexpr (V2) {
            const rsrc_t rwp = make_rsrc(has_wp ? ggw + static_cast<int64_t>(e) * (P * C) : nullptr,
                                         has_wp ? P * C * 4u : 0u);
            static_range<0, NP>([&](auto q) { o.wp[q] = bload<float, kNT>(rwp, off4, (GI.p0 + q) * rowb); });
        }
    };

    auto prologue = [&](int kb, int nb) {
        wave_sync_lds();
        if (lane < nb) {
            const int e = perm[kb + lane];
            const float rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
            float *yp = ylds + lane * DSHP;
            float yv[DSHP], ydv[DSHP];
            if constexpr (!V2) {
                float Y[DSH];
                sh_value<L>(rx, ry, rz, Y);
                static_range<0, DSHP>([&](auto b) {
                    if constexpr (b < DSH)
                        yv[b] = Y[b];
                    else
                        yv[b] = 0.f;
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
                static_range<0, DSHP>([&](auto b) {
                    if constexpr (b < DSH) {
                        yv[b] = Y[b].v;
                        ydv[b] = Y[b].g0 * px + Y[b].g1 * py + Y[b].g2 * pz;
                    } else {
                        yv[b] = 0.f;
                        ydv[b] = 0.f;
                    }
                });
            }
            static_range<0, DSHP / 4>([&](auto q) {
                *reinterpret_cast<float4 *>(yp + 4 * q) =
                    make_float4(yv[4 * q], yv[4 * q + 1], yv[4 * q + 2], yv[4 * q + 3]);
                if constexpr (V2)
                    *reinterpret_cast<float4 *>(yp + B * DSHP + 4 * q) =
                        make_float4(ydv[4 * q], ydv[4 * q + 1], ydv[4 * q + 2], ydv[4 * q + 3]);
            });
        }
        wave_sync_lds();
    };

    // gr / dr of the batch's edges from the parked per-chunk Z sums (lane =
    // edge of the batch, wave 0 only; chunks summed in order).
    auto epilogue = [&](int kb, int nb) {
        __syncthreads();
        if (want_vec && ch == 0 && lane < nb) {
            const int e = perm[kb + lane];
            const float rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
            float z1[DSH], z2[V2 ? DSH : 1];
            static_range<BLO, BHI>([&](auto b) {
                z1[b] = 0.f;
                if constexpr (V2)
                    z2[b] = 0.f;
            });
            for (int c = 0; c < nch; ++c) {
                const float *zp = zall + (sp * nch + c) * (NV * B * DSH) + lane * DSH;
                static_range<BLO, BHI>([&](auto b) {
                    z1[b] += zp[b];
                    if constexpr (V2)
                        z2[b] += zp[B * DSH + b];
                });
            }
            float g0 = 0.f, g1 = 0.f, g2 = 0.f;
            if constexpr (!V2) {
                D3 Y[DSH];
                sh_grad<L>(rx, ry, rz, Y);
                static_range<BLO, BHI>([&](auto b) {
                    g0 = fmaf(z1[b], Y[b].g0, g0);
                    g1 = fmaf(z1[b], Y[b].g1, g1);
                    g2 = fmaf(z1[b], Y[b].g2, g2);
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
                static_range<BLO, BHI>([&](auto b) {
                    g0 = fmaf(z1[b], Y[b].b0, fmaf(z2[b], Y[b].d0, g0));
                    g1 = fmaf(z1[b], Y[b].b1, fmaf(z2[b], Y[b].d1, g1));
                    g2 = fmaf(z1[b], Y[b].b2, fmaf(z2[b], Y[b].d2, g2));
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
        __syncthreads();
    };

    // One edge: per path, the K contraction of the gathered G rows, the node
    // accumulators, the weight cotangent (stored) and the Z partial sums.
    float Z[DSH], Z2[V2 ? DSH : 1];
    static_range<0, DSH>([&](auto b) {
        Z[b] = 0.f;
        if constexpr (V2)
            Z2[b] = 0.f;
    });
    auto compute = [&](const Ops &o, const float *yk, int e) {
        float Yb[DSHP], Ydb[V2 ? DSHP : 1];
        static_range<0, DSHP / 4>([&](auto q) {
            const float4 v = *reinterpret_cast<const float4 *>(yk + 4 * q);
            Yb[4 * q] = v.x;
            Yb[4 * q + 1] = v.y;
            Yb[4 * q + 2] = v.z;
            Yb[4 * q + 3] = v.w;
            if constexpr (V2) {
                const float4 d = *reinterpret_cast<const float4 *>(yk + B * DSHP + 4 * q);
                Ydb[4 * q] = d.x;
                Ydb[4 * q + 1] = d.y;
                Ydb[4 * q + 2] = d.z;
                Ydb[4 * q + 3] = d.w;
            }
        });
        const rsrc_t rgw = make_rsrc(ow ? ow + static_cast<int64_t>(e) * (P * C) : nullptr, ow ? P * C * 4u : 0u);
        static_range<GI.p0, GI.p1>([&](auto p) {
            constexpr Path pa = kTab<L>.path[p];
            constexpr int d1 = 2 * pa.l1 + 1;
            constexpr int XO = pa.x_row - GI.xr0, GO = pa.out_row - GI.gr0, WQ = p - GI.p0;
            const float wp = o.w[WQ];
            float wpp = 0.f;
            if constexpr (V2)
                wpp = o.wp[WQ];
            float wx[d1], xx[V2 ? d1 : 1], s[d1], sd[V2 ? d1 : 1];
            static_range<0, d1>([&](auto a) {
                wx[a] = wp * xr[XO + a];
                if constexpr (V2)
                    xx[a] = fmaf(wp, xpr[XO + a], wpp * xr[XO + a]);
            });
            static_range<kTab<L>.path_ab0[p], kTab<L>.path_ab0[p + 1]>([&](auto g) {
                constexpr ABGroup ag = kTab<L>.ab[g];
                constexpr int a = ag.m1 + pa.l1, b = pa.y_row + pa.l2 + ag.m2;
                float K;
                static_range<ag.t0, ag.t1>([&](auto ti) {
                    constexpr Entry en = kTab<L>.nz[kTab<L>.ab_entries[ti]];
                    if constexpr (ti == ag.t0)
                        K = en.fval * o.g[GO + en.m3 + pa.l3];
                    else
                        K = fmaf(en.fval, o.g[GO + en.m3 + pa.l3], K);
                });
                if constexpr (ab_first_m1(kTab<L>, g)) {
                    s[a] = Yb[b] * K;
                    if constexpr (V2)
                        sd[a] = Ydb[b] * K;
                } else {
                    s[a] = fmaf(Yb[b], K, s[a]);
                    if constexpr (V2)
                        sd[a] = fmaf(Ydb[b], K, sd[a]);
                }
                if constexpr (ab_first_b(kTab<L>, GI.ab0, g)) {
                    if constexpr (V2) {
                        Z[b] = xx[a] * K;
                        Z2[b] = wx[a] * K;
                    } else {
                        Z[b] = wx[a] * K;
                    }
                } else {
                    if constexpr (V2) {
                        Z[b] = fmaf(xx[a], K, Z[b]);
                        Z2[b] = fmaf(wx[a], K, Z2[b]);
                    } else {
                        Z[b] = fmaf(wx[a], K, Z[b]);
                    }
                }
            });
            float gwv;
            static_range<0, d1>([&](auto a) {
                if constexpr (!V2) {
                    acc[XO + a] = fmaf(wp, s[a], acc[XO + a]);
                    if constexpr (a == 0)
                        gwv = xr[XO + a] * s[a];
                    else
                        gwv = fmaf(xr[XO + a], s[a], gwv);
                } else {
                    acc[XO + a] = fmaf(wpp, s[a], fmaf(wp, sd[a], acc[XO + a]));
                    if constexpr (a == 0)
                        gwv = fmaf(xpr[XO + a], s[a], xr[XO + a] * sd[a]);
                    else
                        gwv = fmaf(xpr[XO + a], s[a], fmaf(xr[XO + a], sd[a], gwv));
                }
            });
            bstore<float, kNT>(gwv, rgw, off4, p * rowb);
        });
    };

    // the batch's Z sums: fixed-order DPP wave sum, lane 63 parks them
    auto park_z = [&](int kb) {
        float *zk = zlds + kb * DSH;
        static_range<BLO, BHI>([&](auto b) {
            const float z = wave_sum_to_lane63(Z[b]);
            if (lane == 63)
                zk[b] = z;
            if constexpr (V2) {
                const float z2 = wave_sum_to_lane63(Z2[b]);
                if (lane == 63)
                    zk[B * DSH + b] = z2;
            }
        });
    };

    Ops opA, opB;
    int kb = 0, done = 0;
    if (kb0 < kb1)
        load(kb0, opA);
    for (int k = kb0; k < kb1; k += 2) {
        // edge k uses opA, edge k + 1 uses opB
        {
            const int batch0 = k - kb, nb = min(B, kb1 - batch0);
            if (kb == 0)
                prologue(k, nb);
            if (k + 1 < kb1)
                load(k + 1, opB);
            compute(opA, ylds + kb * DSHP, perm[k]);
            if (want_vec)
                park_z(kb);
            if (++kb == nb) {
                epilogue(batch0, nb);
                kb = 0;
                ++done;
            }
        }
        if (k + 1 >= kb1)
            break;
        {
            const int batch0 = k + 1 - kb, nb = min(B, kb1 - batch0);
            if (kb == 0)
                prologue(k + 1, nb);
            if (k + 2 < kb1)
                load(k + 2, opA);
            compute(opB, ylds + kb * DSHP, perm[k + 1]);
            if (want_vec)
                park_z(kb);
            if (++kb == nb) {
                epilogue(batch0, nb);
                kb = 0;
                ++done;
            }
        }
    }

    // splits with fewer edges still meet every batch barrier
    for (; done < nbatch; ++done)
        epilogue(kb1, 0);

    // the splits' node accumulators meet in wave sp = 0 of each chunk, in order
    if (nsp > 1) {
        __syncthreads();
        if (sp > 0)
            static_range<0, NXR>([&](auto r) { lds[((sp - 1) * nch + ch) * (NXR * 64) + r * 64 + lane] = acc[r]; });
        __syncthreads();
        if (sp == 0)
            for (int q = 1; q < nsp; ++q)
                static_range<0, NXR>([&](auto r) { acc[r] += lds[((q - 1) * nch + ch) * (NXR * 64) + r * 64 + lane]; });
    }

    // node rows of j: stored, or added where the user asked to accumulate or
    // an earlier path group already stored part of the same l1 rows
    if (ox && sp == 0) {
        const rsrc_t rox = make_rsrc(ox + static_cast<int64_t>(j) * (DIN * C), DIN * C * 4u);
        constexpr int L1A = kTab<L>.path[GI.p0].l1;
        constexpr int SHARED_ROWS = GI.shares_first_l1 ? 2 * L1A + 1 : 0;
        const bool acc_all = flags & 1u;
        static_range<0, NXR>([&](auto r) {
            float v = acc[r];
            if (acc_all || r < SHARED_ROWS)
                v += bload<float>(rox, off4, (GI.xr0 + r) * rowb);
            bstore<float>(v, rox, off4, (GI.xr0 + r) * rowb);
        });
    }
}

template <int L, typename XT, int MODE, int SG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ETP_SRC_WPE)))
    src_kernel(const int n_src, const int C, const int *__restrict__ src_ptr, const int *__restrict__ perm,
               const int *__restrict__ perm_dst, const float *__restrict__ vec, const XT *__restrict__ x,
               const float *__restrict__ w, const float *__restrict__ G, const float *__restrict__ ggx,
               const float *__restrict__ ggw, const float *__restrict__ ggvec, float *__restrict__ ox,
               float *__restrict__ ow, float *__restrict__ ovec, const uint32_t flags)
{
    extern __shared__ float lds[];
    src_group<L, XT, MODE, SG>(n_src, C, src_ptr, perm, perm_dst, vec, x, w, G, ggx, ggw, ggvec, ox, ow, ovec, flags,
                               lds);
}

template <int L, typename XT, int MODE>
static hipError_t launch_src_t(const ConvArgs &a)
{
    using Cfg = SrcCfg<L, MODE>;
    constexpr Groups GR = make_src_groups(kTab<L>, Cfg::MAXCOST, Cfg::WMUL);
    const int nch = (a.C + 63) / 64;
    const size_t lds_bytes = sizeof(float) * src_lds_floats<L, MODE>(nch);
    if (a.n_src == 0)
        return hipSuccess;
    hipError_t err = hipSuccess;
    // one launch per path group, in order: later groups add to gr / dr and to
    // the node rows an earlier group started
    static_range<0, GR.n>([&](auto g) {
        if (err != hipSuccess)
            return;
        hipLaunchKernelGGL((src_kernel<L, XT, MODE, g>), dim3(a.n_src), dim3(64 * nch * src_splits(nch)), lds_bytes,
                           a.stream, a.n_src, a.C, a.src_ptr, a.perm, a.perm_dst, a.vec, static_cast<const XT *>(a.x), a.w, a.G, a.ggx,
                           a.ggw, a.ggvec, a.ox, a.ow, a.ovec, a.flags);
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
    return launch_src_t<ETP_L, XT, ETP_MODE>(a);
}

}  // namespace etp
