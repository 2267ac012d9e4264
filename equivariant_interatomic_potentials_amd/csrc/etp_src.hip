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
//     edge split): split s of n takes every n-th of j's out-edges from the
//     s-th on (the out-edges come from the stable transpose of the
//     destination-sorted CSR, so all splits walk the same window of
//     destination rows); a wave's gx / dx rows stay in registers and the
//     splits meet in a fixed-order LDS sum at the end; every wave runs the
//     same number of SH batches so workgroup barriers stay aligned;
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
//     derivatives; no float atomics anywhere;
//   * radial mode (VJP with w = h Wr formed in the kernel): the lane's Wr
//     entries of the group's paths stay in registers, the batch prologue
//     also stores each edge's h row, w is formed at each path's start, and
//     instead of storing gw each lane accumulates gh[k] += gw Wr[k, p, u];
//     the 8 gh sums take the same fixed-order route as gr (wave sum, parked
//     per chunk, chunks in order, later path groups adding to earlier ones);
//   * radial VJP-of-VJP: the same with the cotangent H' on gh as the
//     cotangent W' = H' Wr on gw (formed like w from the edge's H' row), and
//     dw contracted into dh[k] += dw Wr[k, p, u] the way gw becomes gh;
//   * radial weight gradient (modes with WG): each lane also sums, over the
//     node's out-edges, h[e, k] gw[e, p, u] (VJP) or h[e, k] dw[e, p, u] +
//     H'[e, k] gw[e, p, u] (VJP-of-VJP) for its group's paths; the edge
//     splits meet in a fixed-order LDS sum and the node's [8][P][C] block of
//     partials is stored, to be summed over nodes in order afterwards.
#include "etp_conv_common.hpp"

namespace etp {

// Launch shape of the source pass. Per edge a wave keeps in LDS the SH
// values (and for the VJP-of-VJP the directional derivative Yd) and the
// coefficients that turn the Z sums into gr / dr (3 or 6 per SH component);
// B edges per SH batch is the largest power of two up to 64 whose batch fits
// in 8 KiB (16 KiB at two waves per SIMD), so the waves of a CU fit its LDS. MAXCOST bounds the
// registers of one path group (see make_src_groups) and WPE is the waves per
// SIMD the register allocation must allow: four where the group fits in 128
// VGPRs, fewer where the batch's SH (second-order jets at high l_max) need
// more, and two for the VJP-of-VJP, whose groups then take 256 VGPRs (at
// l = 2 all paths fit one group: one walk over the edges instead of four
// beats the lost occupancy, since the pass is VALU-bound and every group
// repeats the SH jets and the x, X' loads). The ETP_SRC_* macros override
// the defaults for tuning builds.
#ifndef ETP_SRC_COST_VJP
#define ETP_SRC_COST_VJP 60
#endif
// VJP-of-VJP contraction order (plain and radial modes): 1 = per (m1, m2) group u, v
// (X' K, x K over m1) and dx += eta K, the SH factors applied per (path, m2)
// afterwards, on the paths where that takes fewer operations; 0 = s, sd and
// Z, Z2 per group on every path
#ifndef ETP_SRC_UV
#define ETP_SRC_UV 1
#endif
#ifndef ETP_SRC_COST_VJP2
#define ETP_SRC_COST_VJP2 100  // one group at l = 2 (two waves per SIMD; 40: four groups, 15% slower)
#endif
#ifndef ETP_SRC_COST_VJP_3
#define ETP_SRC_COST_VJP_3 48  // at three waves per SIMD (32 at four: 5% slower)
#endif
#ifndef ETP_SRC_COST_VJP_4
#define ETP_SRC_COST_VJP_4 40
#endif
#ifndef ETP_SRC_COST_VJP2_3
#define ETP_SRC_COST_VJP2_3 80  // (32 at four waves per SIMD: 13% slower)
#endif
#ifndef ETP_SRC_COST_VJP2_4
#define ETP_SRC_COST_VJP2_4 64  // (40 at three waves per SIMD: 11% slower)
#endif
#ifndef ETP_SRC_COST_RAD
#define ETP_SRC_COST_RAD 150
#endif
#ifndef ETP_SRC_COST_RAD2
#define ETP_SRC_COST_RAD2 120
#endif
#ifndef ETP_SRC_WPE
#define ETP_SRC_WPE 0
#endif
#ifndef ETP_SRC_LDS_BATCH
#define ETP_SRC_LDS_BATCH 8192
#endif
template <int L, int MODE>
struct SrcCfg {
    static constexpr bool WG = MODE == SRC_VJP_RADIAL_WG || MODE == SRC_VJP2_RADIAL_WG;
    static constexpr bool RAD = MODE == SRC_VJP_RADIAL || MODE == SRC_VJP2_RADIAL || WG;
    static constexpr bool V2 = MODE == SRC_VJP2 || MODE == SRC_VJP2_RADIAL || MODE == SRC_VJP2_RADIAL_WG;
    static constexpr int NV = V2 ? 2 : 1;                           // Y (, Yd) and Z (, Z2) copies
    static constexpr int DSH = (L + 1) * (L + 1), DSHP = (DSH + 3) & ~3;
    static constexpr int GQ = 4 * NV * DSH;                         // gr coefficients, a float4 per (b, copy)
    static constexpr int HR = RAD ? (V2 ? 2 : 1) * kRadialMax : 0;  // the edge's h (and H') row (radial modes)
    static constexpr int ES = NV * DSHP + GQ + HR;                  // floats per edge in the batch
    static constexpr int PK = RAD ? 12 : 4;                         // parked sums per edge: gr (, gh), padded
    static constexpr int ESP = ES + 2 * PK;                         // + two park slots
    // at two waves per SIMD (VJP2, radial) a wave may take twice the LDS:
    // longer batches keep more of the prologue's lanes busy (l=3 VJP2: 5%)
    static constexpr int LDS_BATCH = (RAD || V2) ? 2 * ETP_SRC_LDS_BATCH : ETP_SRC_LDS_BATCH;
    static constexpr int B = [] {
        int b = 64;
        while (b > 8 && b * ESP * 4 > LDS_BATCH)
            b >>= 1;
        return b;
    }();
    // registers per path beyond its G rows: the w row (and W'), or in the
    // radial mode the 8 Wr entries
    static constexpr int WMUL = RAD ? (WG ? 2 : 1) * kRadialMax : (V2 ? 2 : 1);
    static constexpr int MAXCOST = RAD ? (V2 ? (L <= 2 ? ETP_SRC_COST_RAD2 : L == 3 ? 100 : 80)
                                             : (L <= 2 ? ETP_SRC_COST_RAD : L == 3 ? 130 : 100))
                                   : V2 ? (L <= 2 ? ETP_SRC_COST_VJP2 : L == 3 ? ETP_SRC_COST_VJP2_3
                                                                             : ETP_SRC_COST_VJP2_4)
                                                      : (L <= 2 ? ETP_SRC_COST_VJP : L == 3 ? ETP_SRC_COST_VJP_3
                                                                                         : ETP_SRC_COST_VJP_4);
    static constexpr int WPE = ETP_SRC_WPE > 0 ? ETP_SRC_WPE : (RAD || V2) ? 2 : (L == 3 ? 3 : 4);
};

// Edge splits per channel chunk: four waves per workgroup in total.
constexpr int src_splits(int nch) { return nch >= 4 ? 1 : 4 / nch; }

template <int L, int MODE>
constexpr int src_lds_floats(int nch)
{
    using Cfg = SrcCfg<L, MODE>;
    const int nw = nch * src_splits(nch);
    // per wave: the batch (B x ES) and two alternating park slots (B x PK)
    const int batch = nw * Cfg::B * Cfg::ESP;
    int rows = kTab<L>.din_rows;  // node rows of the splits (and the weight-gradient partials)
    if (Cfg::WG) {
        const Groups GR = make_src_groups(kTab<L>, Cfg::MAXCOST, Cfg::WMUL);
        for (int k = 0; k < GR.n; ++k) {
            const int np = (GR.p1[k] - GR.p0[k]) * kRadialMax;
            rows = np > rows ? np : rows;
        }
    }
    const int reduce = (src_splits(nch) - 1) * nch * rows * 64;
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
                                          const uint32_t flags, float *lds, const float *__restrict__ hrad,
                                          const float *__restrict__ wrad, const int nbasis,
                                          float *__restrict__ oh, const float *__restrict__ ggh,
                                          float *__restrict__ owr)
{
    using Cfg = SrcCfg<L, MODE>;
    constexpr int B = Cfg::B, ES = Cfg::ES, NV = Cfg::NV, DSHP = Cfg::DSHP, PK = Cfg::PK;
    constexpr bool V2 = Cfg::V2, RAD = Cfg::RAD, WG = Cfg::WG;
    constexpr int RK = kRadialMax, HO = NV * DSHP + Cfg::GQ;  // h row offset in an edge's batch slot
    constexpr Groups GR = make_src_groups(kTab<L>, Cfg::MAXCOST, Cfg::WMUL);
    constexpr SrcGroupInfo GI = src_group_info(kTab<L>, GR, SG);
    constexpr int P = kTab<L>.P, DIN = kTab<L>.din_rows, DOUT = kTab<L>.dout_rows, DSH = kTab<L>.dsh;
    constexpr int NP = GI.np, NXR = GI.nxr, NGR = GI.ngr;
    constexpr int BLO = sh_lo(kTab<L>, GI.p0, GI.p1), BHI = sh_hi(kTab<L>, GI.p0, GI.p1);

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
    const bool want_vec = ovec != nullptr, want_h = RAD && oh != nullptr;
    const bool has_xp = V2 && ggx != nullptr, has_rp = V2 && ggvec != nullptr;
    // W' comes from memory, or in the radial mode from the edge's H' row
    const bool has_wp = V2 && (RAD ? ggh != nullptr : ggw != nullptr);
    const uint32_t rowb = static_cast<uint32_t>(C) * 4u;

    // LDS: per wave the batch [B][ES] and two park slots [2][B][PK]
    const int nw = nch * nsp;
    float *blds = lds + wv * (B * ES);
    float *pall = lds + nw * (B * ES);
    float *plds = pall + wv * (2 * B * PK);

    // this wave's split of j's out-edges: every nsp-th edge from sp on, so
    // that the splits walk the same (destination-ordered) window of G rows;
    // every wave runs nbatch batches
    const int kbase = src_ptr[j] + sp, len = src_ptr[j + 1] - src_ptr[j];
    const int cnt = len > sp ? (len - sp + nsp - 1) / nsp : 0;
    const int nbatch = ((len + nsp - 1) / nsp + B - 1) / B;
    auto kpos = [&](int i) { return kbase + i * nsp; };  // position of the split's i-th edge

    // radial mode: the lane's Wr[k, p, u] for the group's paths (zero past
    // nbasis and C)
    float wr[RAD ? NP : 1][RK];
    if constexpr (RAD) {
        static_range<0, NP>([&](auto q) {
            static_range<0, RK>([&](auto k) {
                wr[q][k] =
                    (active && k < nbasis) ? wrad[(static_cast<int64_t>(k) * P + GI.p0 + q) * C + u] : 0.f;
            });
        });
    }

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

    // Operands of one edge, per path of the group: the w (and W') row and
    // the path's own G[i] rows. Rows of different paths are disjoint, so a
    // path's registers are reloaded with the next edge's rows as soon as the
    // path is done: one edge of look-ahead without a second register set.
    struct Ops {
        float w[NP], wp[V2 ? NP : 1], g[NGR];
    };
    struct EdgeRsrc {
        rsrc_t w, wp, g;
    };
    auto edge_rsrc = [&](int k, bool valid) {
        const int e = perm[k], i = perm_dst[k];
        EdgeRsrc r;
        r.w = make_rsrc(RAD ? nullptr : w + static_cast<int64_t>(e) * (P * C), (!RAD && valid) ? P * C * 4u : 0u);
        r.g = make_rsrc(G + static_cast<int64_t>(i) * (DOUT * C), valid ? DOUT * C * 4u : 0u);
        r.wp = make_rsrc((has_wp && !RAD) ? ggw + static_cast<int64_t>(e) * (P * C) : nullptr,
                         (has_wp && !RAD && valid) ? P * C * 4u : 0u);
        return r;
    };
    Ops o;
    auto load_path = [&](auto p, const EdgeRsrc &r) {
        constexpr Path pa = kTab<L>.path[p];
        constexpr int GO = pa.out_row - GI.gr0, WQ = p - GI.p0;
        if constexpr (!RAD)  // (the radial mode forms w at the path's start)
            o.w[WQ] = bload<float, kNT>(r.w, off4, p * rowb);
        if constexpr (V2 && !RAD)
            o.wp[WQ] = bload<float, kNT>(r.wp, off4, p * rowb);
        static_range<0, 2 * pa.l3 + 1>([&](auto m) { o.g[GO + m] = bload<float>(r.g, off4, (pa.out_row + m) * rowb); });
    };

    // Per batch, lane = edge: Y (, Yd) and the coefficients of the gr / dr
    // contraction, dY_b/dr (VJP) or the two Hessian-vector terms (VJP2).
    auto prologue = [&](int i0, int nb) {
        wave_sync_lds();
        if (lane < nb) {
            const int e = perm[kpos(i0 + lane)];
            const float rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
            float *ep = blds + lane * ES;
            float4 *cp = reinterpret_cast<float4 *>(ep + NV * DSHP);
            // padding of the SH rows (the edge loop reads them as float4)
            static_range<DSH, DSHP>([&](auto b) {
                ep[b] = 0.f;
                if constexpr (V2)
                    ep[DSHP + b] = 0.f;
            });
            if constexpr (!V2) {
                sh_grad_emit<L>(rx, ry, rz, [&](auto b, const D3 &y) {
                    ep[b] = y.v;
                    cp[b] = make_float4(y.g0, y.g1, y.g2, 0.f);
                });
                if constexpr (RAD)
                    static_range<0, RK>([&](auto k) {
                        ep[HO + k] = k < nbasis ? hrad[static_cast<int64_t>(e) * nbasis + k] : 0.f;
                    });
            } else {
                float px = 0.f, py = 0.f, pz = 0.f;
                if (has_rp) {
                    px = ggvec[3 * e];
                    py = ggvec[3 * e + 1];
                    pz = ggvec[3 * e + 2];
                }
                sh_jet_emit<L>(rx, ry, rz, px, py, pz, [&](auto b, const Jet &y) {
                    ep[b] = y.a;
                    ep[DSHP + b] = y.c;
                    cp[2 * b] = make_float4(y.b0, y.b1, y.b2, 0.f);
                    cp[2 * b + 1] = make_float4(y.d0, y.d1, y.d2, 0.f);
                });
                if constexpr (RAD)
                    static_range<0, RK>([&](auto k) {
                        ep[HO + k] = k < nbasis ? hrad[static_cast<int64_t>(e) * nbasis + k] : 0.f;
                        ep[HO + RK + k] = (has_wp && k < nbasis) ? ggh[static_cast<int64_t>(e) * nbasis + k] : 0.f;
                    });
            }
        }
        wave_sync_lds();
    };

    // gr / dr of a finished batch from the parked per-chunk partial sums
    // (several chunks only): lane = edge of the batch, chunk 0's wave of the
    // split adds the chunks in order. The park slots alternate by batch, so
    // one barrier per batch keeps writers and the reader apart.
    auto epilogue = [&](int i0, int nb, int slot) {
        __syncthreads();
        if (want_vec && ch == 0 && lane < nb) {
            float g0 = 0.f, g1 = 0.f, g2 = 0.f;
            for (int c = 0; c < nch; ++c) {
                const float *pp = pall + (sp * nch + c) * (2 * B * PK) + (slot * B + lane) * PK;
                g0 += pp[0];
                g1 += pp[1];
                g2 += pp[2];
            }
            float *gp = ovec + 3 * static_cast<int64_t>(perm[kpos(i0 + lane)]);
            if (SG > 0) {  // later source groups add to the earlier groups' result
                g0 += gp[0];
                g1 += gp[1];
                g2 += gp[2];
            }
            gp[0] = g0;
            gp[1] = g1;
            gp[2] = g2;
        }
        if constexpr (RAD) {
            if (want_h && ch == 0 && lane < nb) {
                float gk[RK];
                static_range<0, RK>([&](auto k) { gk[k] = 0.f; });
                for (int c = 0; c < nch; ++c) {
                    const float *pp = pall + (sp * nch + c) * (2 * B * PK) + (slot * B + lane) * PK + 4;
                    static_range<0, RK>([&](auto k) { gk[k] += pp[k]; });
                }
                float *hp = oh + static_cast<int64_t>(perm[kpos(i0 + lane)]) * nbasis;
                static_range<0, RK>([&](auto k) {
                    if (k < nbasis)
                        hp[k] = SG > 0 ? hp[k] + gk[k] : gk[k];
                });
            }
        }
    };

    // One edge, path by path: the K contraction of the gathered G rows, the
    // node accumulators, the weight cotangent (stored) and the Z partial
    // sums; then the path's registers take the next edge's rows.
    float Z[DSH], Z2[V2 ? DSH : 1], ghk[RAD ? RK : 1];
    // the weight-gradient sums of the group's paths over the node's out-edges
    float wg[WG ? NP : 1][WG ? RK : 1];
    if constexpr (WG)
        static_range<0, NP>([&](auto q) { static_range<0, RK>([&](auto k) { wg[q][k] = 0.f; }); });
    static_range<0, DSH>([&](auto b) {
        Z[b] = 0.f;
        if constexpr (V2)
            Z2[b] = 0.f;
    });
    auto compute = [&](const float *ep, int e, const EdgeRsrc &nx) {
        float Yb[DSHP], Ydb[V2 ? DSHP : 1];
        static_range<0, DSHP / 4>([&](auto q) {
            const float4 v = *reinterpret_cast<const float4 *>(ep + 4 * q);
            Yb[4 * q] = v.x;
            Yb[4 * q + 1] = v.y;
            Yb[4 * q + 2] = v.z;
            Yb[4 * q + 3] = v.w;
            if constexpr (V2) {
                const float4 d = *reinterpret_cast<const float4 *>(ep + DSHP + 4 * q);
                Ydb[4 * q] = d.x;
                Ydb[4 * q + 1] = d.y;
                Ydb[4 * q + 2] = d.z;
                Ydb[4 * q + 3] = d.w;
            }
        });
        const rsrc_t rgw = make_rsrc(ow ? ow + static_cast<int64_t>(e) * (P * C) : nullptr, ow ? P * C * 4u : 0u);
        float4 h0, h1, hp0, hp1;
        if constexpr (RAD) {
            h0 = *reinterpret_cast<const float4 *>(ep + HO);
            h1 = *reinterpret_cast<const float4 *>(ep + HO + 4);
            if constexpr (V2) {
                hp0 = *reinterpret_cast<const float4 *>(ep + HO + RK);
                hp1 = *reinterpret_cast<const float4 *>(ep + HO + RK + 4);
            }
            static_range<0, RK>([&](auto k) { ghk[k] = 0.f; });
        }
        // the radial weight of path slot q: sum_k a[k] Wr[k, p, u], k in order
        // (a = the edge's h row for w, its H' row for W')
        auto wr_dot = [&](auto q, const float4 &a0, const float4 &a1) {
            float t = a0.x * wr[q][0];
            t = fmaf(a0.y, wr[q][1], t);
            t = fmaf(a0.z, wr[q][2], t);
            t = fmaf(a0.w, wr[q][3], t);
            t = fmaf(a1.x, wr[q][4], t);
            t = fmaf(a1.y, wr[q][5], t);
            t = fmaf(a1.z, wr[q][6], t);
            return fmaf(a1.w, wr[q][7], t);
        };
        // VJP-of-VJP of one path in the order with one FMA fewer per (m1, m2)
        // group: u[b] = sum_a X'[a] K, v[b] = sum_a x[a] K, eta[b] = W' Y_b + w Yd_b;
        // dx[a] += eta[b] K per group, then per (path, b) used
        //   dw = sum_b Y_b u[b] + Yd_b v[b],  Z[b] += w u[b] + W' v[b],  Z2[b] += w v[b]
        // (the sums of s, sd, xx and wx below, regrouped)
        auto path_uv = [&](auto p) {
            constexpr Path pa = kTab<L>.path[p];
            constexpr int d2 = 2 * pa.l2 + 1, YB = pa.y_row;
            constexpr int XO = pa.x_row - GI.xr0, GO = pa.out_row - GI.gr0, WQ = p - GI.p0;
            constexpr int PA0 = kTab<L>.path_ab0[p], PA1 = kTab<L>.path_ab0[p + 1];
            float wp, wpp;
            if constexpr (RAD) {
                wp = wr_dot(ic<WQ>{}, h0, h1);
                wpp = wr_dot(ic<WQ>{}, hp0, hp1);
            } else {
                wp = o.w[WQ];
                wpp = o.wp[WQ];
            }
            float eta[d2], u[d2], v[d2];
            static_range<0, d2>([&](auto m) {
                if constexpr (ab_touches_b(kTab<L>, PA0, PA1, YB + m))
                    eta[m] = fmaf(wp, Ydb[YB + m], wpp * Yb[YB + m]);
            });
            static_range<PA0, PA1>([&](auto g) {
                constexpr ABGroup ag = kTab<L>.ab[g];
                constexpr int a = ag.m1 + pa.l1, m = pa.l2 + ag.m2;
                float K;
                static_range<ag.t0, ag.t1>([&](auto ti) {
                    constexpr Entry en = kTab<L>.nz[kTab<L>.ab_entries[ti]];
                    if constexpr (ti == ag.t0)
                        K = en.fval * o.g[GO + en.m3 + pa.l3];
                    else
                        K = fmaf(en.fval, o.g[GO + en.m3 + pa.l3], K);
                });
                if constexpr (ab_first_b(kTab<L>, PA0, g)) {
                    u[m] = xpr[XO + a] * K;
                    v[m] = xr[XO + a] * K;
                } else {
                    u[m] = fmaf(xpr[XO + a], K, u[m]);
                    v[m] = fmaf(xr[XO + a], K, v[m]);
                }
                acc[XO + a] = fmaf(eta[m], K, acc[XO + a]);
            });
            load_path(p, nx);
            float gwv = 0.f;
            bool started = false;
            static_range<0, d2>([&](auto m) {
                constexpr int b = YB + m;
                if constexpr (ab_touches_b(kTab<L>, PA0, PA1, b)) {
                    gwv = started ? fmaf(Yb[b], u[m], fmaf(Ydb[b], v[m], gwv)) : fmaf(Yb[b], u[m], Ydb[b] * v[m]);
                    started = true;
                    if constexpr (!ab_touches_b(kTab<L>, GI.ab0, PA0, b)) {  // b's first path in the group
                        Z[b] = fmaf(wp, u[m], wpp * v[m]);
                        Z2[b] = wp * v[m];
                    } else {
                        Z[b] = fmaf(wp, u[m], fmaf(wpp, v[m], Z[b]));
                        Z2[b] = fmaf(wp, v[m], Z2[b]);
                    }
                }
            });
            if constexpr (RAD)  // d_h[e, k] += d_w[e, p, u] Wr[k, p, u] (summed over lanes later)
                static_range<0, RK>([&](auto k) { ghk[k] = fmaf(gwv, wr[WQ][k], ghk[k]); });
            else
                bstore<float, kNT>(gwv, rgw, off4, p * rowb);
            if constexpr (WG) {
                // dWr[k, p, u] += h[e, k] dw + H'[e, k] gw, with the plain
                // gw = sum_m1 x s = sum_b Y_b v[b]
                float gpl = 0.f;
                static_range<0, d2>([&](auto m) {
                    if constexpr (ab_touches_b(kTab<L>, PA0, PA1, YB + m))
                        gpl = fmaf(Yb[YB + m], v[m], gpl);
                });
                const float hk[RK] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                const float hpk[RK] = {hp0.x, hp0.y, hp0.z, hp0.w, hp1.x, hp1.y, hp1.z, hp1.w};
                static_range<0, RK>([&](auto k) { wg[WQ][k] = fmaf(hpk[k], gpl, fmaf(hk[k], gwv, wg[WQ][k])); });
            }
        };
        static_range<GI.p0, GI.p1>([&](auto p) {
#ifdef ETP_SRC_SCHED_FENCE
            __builtin_amdgcn_sched_barrier(0);
#endif
            // (at l_max = 3 only without radial weights and on paths whose u, v,
            // eta take no more registers than s, sd, wx, xx; at l_max = 4 on
            // none: the larger path groups spill either way)
            if constexpr (V2 && ETP_SRC_UV && uv_cheaper(kTab<L>, p) &&
                          (L <= 2 || (L == 3 && !RAD &&
                                      3 * (2 * kTab<L>.path[p].l2 + 1) <= 4 * (2 * kTab<L>.path[p].l1 + 1)))) {
                path_uv(p);
                return;
            }
            constexpr Path pa = kTab<L>.path[p];
            constexpr int d1 = 2 * pa.l1 + 1;
            constexpr int XO = pa.x_row - GI.xr0, GO = pa.out_row - GI.gr0, WQ = p - GI.p0;
            float wp;
            if constexpr (RAD)  // w[e, p, u] = sum_k h[e, k] Wr[k, p, u]
                wp = wr_dot(ic<WQ>{}, h0, h1);
            else
                wp = o.w[WQ];
            float wpp = 0.f;
            if constexpr (V2 && RAD)  // W'[e, p, u] = sum_k H'[e, k] Wr[k, p, u]
                wpp = wr_dot(ic<WQ>{}, hp0, hp1);
            else if constexpr (V2)
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
            load_path(p, nx);
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
            if constexpr (RAD)  // gh[e, k] += gw[e, p, u] Wr[k, p, u] (summed over lanes later)
                static_range<0, RK>([&](auto k) { ghk[k] = fmaf(gwv, wr[WQ][k], ghk[k]); });
            else
                bstore<float, kNT>(gwv, rgw, off4, p * rowb);
            if constexpr (WG) {
                // dWr[k, p, u] += h[e, k] gw (VJP), or h[e, k] dw + H'[e, k] gw
                // with the plain gw = sum_m1 x s (VJP-of-VJP)
                const float hk[RK] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                if constexpr (V2) {
                    float gpl = 0.f;
                    static_range<0, d1>([&](auto a) { gpl = fmaf(xr[XO + a], s[a], gpl); });
                    const float hpk[RK] = {hp0.x, hp0.y, hp0.z, hp0.w, hp1.x, hp1.y, hp1.z, hp1.w};
                    static_range<0, RK>([&](auto k) { wg[WQ][k] = fmaf(hpk[k], gpl, fmaf(hk[k], gwv, wg[WQ][k])); });
                } else {
                    static_range<0, RK>([&](auto k) { wg[WQ][k] = fmaf(hk[k], gwv, wg[WQ][k]); });
                }
            }
        });
    };

    // The edge's gr / dr partial over this wave's channels: Z contracted
    // with the edge's coefficients per lane, then a fixed-order DPP sum of
    // the three components (the sum is exact in lane 63).
    auto fold = [&](const float *ep, float &g0, float &g1, float &g2) {
        const float4 *cp = reinterpret_cast<const float4 *>(ep + NV * DSHP);
        g0 = 0.f;
        g1 = 0.f;
        g2 = 0.f;
        static_range<BLO, BHI>([&](auto b) {
            const float4 c = cp[NV * b];
            g0 = fmaf(Z[b], c.x, g0);
            g1 = fmaf(Z[b], c.y, g1);
            g2 = fmaf(Z[b], c.z, g2);
            if constexpr (V2) {
                const float4 d = cp[2 * b + 1];
                g0 = fmaf(Z2[b], d.x, g0);
                g1 = fmaf(Z2[b], d.y, g1);
                g2 = fmaf(Z2[b], d.z, g2);
            }
        });
        g0 = wave_sum_to_lane63(g0);
        g1 = wave_sum_to_lane63(g1);
        g2 = wave_sum_to_lane63(g2);
        if constexpr (RAD)
            static_range<0, RK>([&](auto k) { ghk[k] = wave_sum_to_lane63(ghk[k]); });
    };

    int kb = 0, done = 0;
    static_range<0, NXR>([&](auto q) {
        settle(xr[q]);
        if constexpr (V2)
            settle(xpr[q]);
    });
    for (int i = 0; i < cnt; ++i) {
        const int batch0 = i - kb, nb = min(B, cnt - batch0), k = kpos(i);
        if (kb == 0) {
            // the look-ahead stops at batch ends, so no operand registers
            // are live while the batch's SH are evaluated
            prologue(i, nb);
            const EdgeRsrc r0 = edge_rsrc(k, true);
            static_range<GI.p0, GI.p1>([&](auto p) { load_path(p, r0); });
        }
        const bool more = kb + 1 < nb;
        const EdgeRsrc nx = edge_rsrc(more ? k + nsp : k, more);
        const int e = perm[k];
        const float *ep = blds + kb * ES;
        compute(ep, e, nx);
        // the fold runs whether or not gr / dr is wanted: guarding it lets the
        // compiler sink the Z sums into the branch and keep every K alive
        float g0, g1, g2;
        fold(ep, g0, g1, g2);
        if (want_vec) {
            if (nch == 1) {
                // one chunk: lane 63 holds the edge's whole sum
                if (lane == 63) {
                    float *gp = ovec + 3 * static_cast<int64_t>(e);
                    if (SG > 0) {
                        g0 += gp[0];
                        g1 += gp[1];
                        g2 += gp[2];
                    }
                    gp[0] = g0;
                    gp[1] = g1;
                    gp[2] = g2;
                }
            } else if (lane == 63) {
                float *pp = plds + ((done & 1) * B + kb) * PK;
                pp[0] = g0;
                pp[1] = g1;
                pp[2] = g2;
            }
        }
        if constexpr (RAD) {
            if (want_h && lane == 63) {
                if (nch == 1) {
                    float *hp = oh + static_cast<int64_t>(e) * nbasis;
                    static_range<0, RK>([&](auto k) {
                        if (k < nbasis)
                            hp[k] = SG > 0 ? hp[k] + ghk[k] : ghk[k];
                    });
                } else {
                    float *pp = plds + ((done & 1) * B + kb) * PK + 4;
                    static_range<0, RK>([&](auto k) { pp[k] = ghk[k]; });
                }
            }
        }
        if (++kb == nb) {
            if (nch > 1)
                epilogue(batch0, nb, done & 1);
            kb = 0;
            ++done;
        }
    }

    // splits with fewer edges still meet every batch barrier
    if (nch > 1)
        for (; done < nbatch; ++done)
            epilogue(cnt, 0, done & 1);

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

    // the weight-gradient partials: the splits meet in wave sp = 0 of each
    // chunk, in order, and node j's block [8][P][C] (this group's paths) is
    // stored
    if constexpr (WG) {
        if (nsp > 1) {
            constexpr int NR = NP * RK;
            __syncthreads();
            if (sp > 0)
                static_range<0, NP>([&](auto q) {
                    static_range<0, RK>([&](auto k) {
                        lds[((sp - 1) * nch + ch) * (NR * 64) + (q * RK + k) * 64 + lane] = wg[q][k];
                    });
                });
            __syncthreads();
            if (sp == 0)
                for (int t = 1; t < nsp; ++t)
                    static_range<0, NP>([&](auto q) {
                        static_range<0, RK>([&](auto k) {
                            wg[q][k] += lds[((t - 1) * nch + ch) * (NR * 64) + (q * RK + k) * 64 + lane];
                        });
                    });
        }
        if (owr && sp == 0) {
            const rsrc_t rw = make_rsrc(owr + static_cast<int64_t>(j) * (RK * P * C), RK * P * C * 4u);
            static_range<0, NP>([&](auto q) {
                static_range<0, RK>([&](auto k) { bstore<float>(wg[q][k], rw, off4, (k * P + GI.p0 + q) * rowb); });
            });
        }
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
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SrcCfg<L, MODE>::WPE)))
    src_kernel(const int n_src, const int C, const int *__restrict__ src_ptr, const int *__restrict__ perm,
               const int *__restrict__ perm_dst, const float *__restrict__ vec, const XT *__restrict__ x,
               const float *__restrict__ w, const float *__restrict__ G, const float *__restrict__ ggx,
               const float *__restrict__ ggw, const float *__restrict__ ggvec, float *__restrict__ ox,
               float *__restrict__ ow, float *__restrict__ ovec, const uint32_t flags,
               const float *__restrict__ hrad, const float *__restrict__ wrad, const int nbasis,
               float *__restrict__ oh, const float *__restrict__ ggh, float *__restrict__ owr)
{
    extern __shared__ float lds[];
    src_group<L, XT, MODE, SG>(n_src, C, src_ptr, perm, perm_dst, vec, x, w, G, ggx, ggw, ggvec, ox, ow, ovec, flags,
                               lds, hrad, wrad, nbasis, oh, ggh, owr);
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
                           a.ggw, a.ggvec, a.ox, a.ow, a.ovec, a.flags, a.h, a.wr, a.nbasis, a.oh, a.ggh, a.owr);
        err = hipGetLastError();
    });
    return err;
}

#if !defined(ETP_L) || !defined(ETP_XT) || !defined(ETP_MODE)
#error "compile this file once per (l_max, dtype, mode) with -DETP_L=0..4 -DETP_XT=0|1 -DETP_MODE=0..5"
#endif

hipError_t ETP_RUN_NAME(src, ETP_L, ETP_XT, ETP_MODE)(const ConvArgs &a)
{
    using XT = std::conditional_t<ETP_XT == 1, bf16raw, float>;
    return launch_src_t<ETP_L, XT, ETP_MODE>(a);
}

}  // namespace etp
