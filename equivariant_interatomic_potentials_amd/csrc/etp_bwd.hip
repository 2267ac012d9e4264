// etp_bwd.hip -- destination-segmented backward of the edge tensor-product
// convolution: the VJP (forces) and the VJP-of-VJP (force training) walked
// over each destination's in-edges, so that the cotangent rows G[i] (Dout
// rows per node, the widest operand of the backward) are read once per node
// and stay in registers, while each edge gathers only its source's Din rows of
// x. The convolution's cost is memory access and edge aggregation rather than
// arithmetic ("How does FlashCart make equivariant interatomic potentials
// faster and more accurate?", section "Cartesian kernels replace SH
// coupling"; the VJP and VJP-of-VJP are the stages measured in its section
// "Generated kernels beat SH baselines at high order").
//
// For edge e = (i <- j), with K[p, m1, m2] = sum_m3 C G[i, p, m3]:
//   VJP   part[e, m1]  = sum_p w s[m1],            s[m1] = sum_m2 Y_m2 K[m1, m2]
//         gw[e, p]     = sum_m1 x[j, m1] s[m1]
//         gr[e]        = sum_b Z_b dY_b/dr,       Z_b   = sum_{p,u,m1} w x[j, m1] K[m1, b]
//   VJP2  part[e, m1]  = sum_p W' s[m1] + w sd[m1],  sd[m1] = sum_m2 Yd_m2 K[m1, m2]
//         dw[e, p]     = sum_m1 X'[m1] s[m1] + x[m1] sd[m1]
//         dr[e]        = sum_b Z1_b dY_b/dr + Z2_b d(grad Y_b . R')/dr
//   with Yd = grad Y . R', Z1_b = sum (w X' + W' x) K, Z2_b = sum w x K (the
//   VJP-of-VJP's dG is the destination pass of etp_dst.hip, which needs no
//   G). The node gradient gx (dx) is the sum of part
//   over each source's out-edges, which a second kernel forms in the order of
//   the stable transpose (fixed order: deterministic, no atomics):
//         gx[j] = sum_{k in [src_ptr[j], src_ptr[j+1])} part[perm[k]].
//
// Mapping (gfx950, wave64):
//   * one workgroup per destination node i and path group (groups are
//     successive launches), one wave per (64-channel chunk, edge split);
//     split s of n takes every n-th in-edge from the s-th on;
//   * the group's G[i] rows stay in registers for the whole node; per edge
//     the wave streams the w (W') rows of the group's paths and gathers the x
//     (X') rows of its l1 values, one edge of look-ahead in one register set;
//   * per batch of B edges lane k evaluates the SH of edge k (and the
//     coefficients of the gr / dr contraction) into the wave's LDS slice,
//     read back as broadcasts;
//   * part rows of an l1 block are stored as soon as the block's last path of
//     the group is done (a group that starts inside an l1 block adds to the
//     rows the previous group stored); gw / dw rows are stored per path;
//   * Z is reduced over each wave's lanes with DPP in a fixed order, parked
//     in LDS per chunk, and chunk 0's wave adds the chunks in order and turns
//     them into gr / dr; later path groups add to the earlier groups' result.
#include "etp_conv_common.hpp"

namespace etp {

enum { BWD_VJP = 0, BWD_VJP2 = 1 };

#ifndef ETP_BWD_COST_VJP
#define ETP_BWD_COST_VJP 96
#endif
#ifndef ETP_BWD_COST_VJP_3
#define ETP_BWD_COST_VJP_3 96
#endif
#ifndef ETP_BWD_COST_VJP_4
#define ETP_BWD_COST_VJP_4 56
#endif
#ifndef ETP_BWD_COST_VJP2
#define ETP_BWD_COST_VJP2 160
#endif
#ifndef ETP_BWD_COST_VJP2_3
#define ETP_BWD_COST_VJP2_3 100
#endif
#ifndef ETP_BWD_COST_VJP2_4
#define ETP_BWD_COST_VJP2_4 64
#endif
#ifndef ETP_BWD_WPE_VJP
#define ETP_BWD_WPE_VJP 2
#endif
#ifndef ETP_BWD_WPE_VJP2
#define ETP_BWD_WPE_VJP2 2
#endif
#ifndef ETP_BWD_LDS_BATCH
#define ETP_BWD_LDS_BATCH 16384
#endif
// VJP-of-VJP contraction order: 1 = per (m1, m2) group the three products
// u, v (X' K, x K over m1) and part += eta K, the SH factors applied per
// (path, m2) afterwards, on the paths where that takes fewer operations;
// 0 = s, sd (Y K, Yd K over m2) and Z, Z2 per group on every path
#ifndef ETP_BWD_UV
#define ETP_BWD_UV 1
#endif

// Path groups of the destination-side backward: contiguous paths whose
// registers fit: gmul per resident G row (G, and dG for the VJP-of-VJP),
// wmul per path (w, W'), xmul per x row (x, X' and the partial sums).
// Whole l1 blocks are kept together while they fit (their part rows are then
// written once); a block that alone exceeds the bound is cut at path
// boundaries.
constexpr int bwd_cost(const Table &T, int p0, int p1, int gmul, int wmul, int xmul)
{
    const int l1a = T.path[p0].l1, l1b = T.path[p1 - 1].l1;
    const int xrows = (l1b + 1) * (l1b + 1) - l1a * l1a;
    const int grows = T.path[p1 - 1].out_row + 2 * T.path[p1 - 1].l3 + 1 - T.path[p0].out_row;
    return gmul * grows + wmul * (p1 - p0) + xmul * xrows;
}

constexpr Groups make_bwd_groups(const Table &T, int max_cost, int gmul, int wmul, int xmul)
{
    Groups g{};
    int start = 0, p = 0;
    while (p < T.P) {
        int b1 = p;  // end of the l1 block that starts at p
        while (b1 < T.P && T.path[b1].l1 == T.path[p].l1)
            ++b1;
        if (bwd_cost(T, start, b1, gmul, wmul, xmul) <= max_cost) {
            p = b1;
            continue;
        }
        if (start < p) {  // close the group before this block
            g.p0[g.n] = start;
            g.p1[g.n] = p;
            ++g.n;
            start = p;
            if (bwd_cost(T, start, b1, gmul, wmul, xmul) <= max_cost) {
                p = b1;
                continue;
            }
        }
        // the block alone is too big: cut it at path boundaries
        for (int q = p + 1; q <= b1; ++q) {
            if (q == b1 || bwd_cost(T, start, q + 1, gmul, wmul, xmul) > max_cost) {
                if (q == b1)
                    break;
                g.p0[g.n] = start;
                g.p1[g.n] = q;
                ++g.n;
                start = q;
            }
        }
        p = b1;
    }
    g.p0[g.n] = start;
    g.p1[g.n] = T.P;
    ++g.n;
    return g;
}

template <int L, int MODE>
struct BwdCfg {
    static constexpr bool V2 = MODE == BWD_VJP2;
    static constexpr int NV = V2 ? 2 : 1;                          // Y (, Yd) and Z (, Z2) copies
    static constexpr int DSH = (L + 1) * (L + 1), DSHP = (DSH + 3) & ~3;
    static constexpr int GQ = 4 * NV * DSH;                        // gr coefficients, a float4 per (b, copy)
    static constexpr int GMUL = 1, WMUL = V2 ? 2 : 1, XMUL = V2 ? 3 : 2;
    // the bound counts the group's own registers; the SH-sized arrays (Y, Z)
    // come on top, so it shrinks with l_max
    static constexpr int MAXCOST = V2 ? (L <= 2 ? ETP_BWD_COST_VJP2 : L == 3 ? ETP_BWD_COST_VJP2_3 : ETP_BWD_COST_VJP2_4)
                                      : (L <= 2 ? ETP_BWD_COST_VJP : L == 3 ? ETP_BWD_COST_VJP_3 : ETP_BWD_COST_VJP_4);
    static constexpr Groups GR = make_bwd_groups(kTab<L>, MAXCOST, GMUL, WMUL, XMUL);
    static constexpr int ES = NV * DSHP + GQ;                       // floats per edge in the batch
    static constexpr int PK = 4;                                    // parked gr sums per edge, padded
    static constexpr int ESP = ES + 2 * PK;
    static constexpr int B = [] {
        int b = 64;
        while (b > 4 && b * ESP * 4 > ETP_BWD_LDS_BATCH)
            b >>= 1;
        return b;
    }();
    static constexpr int WPE = V2 ? ETP_BWD_WPE_VJP2 : ETP_BWD_WPE_VJP;
};

// Whether paths a and b (both in range) have the same l1.
constexpr bool same_l1(const Table &T, int a, int b)
{
    return a >= 0 && b < T.P && T.path[a].l1 == T.path[b].l1;
}

// Waves per workgroup: 64-channel chunks x edge splits, four in all.
constexpr int bwd_splits(int nch) { return nch >= 4 ? 1 : 4 / nch; }

template <int L, int MODE>
constexpr int bwd_lds_floats(int nch)
{
    using Cfg = BwdCfg<L, MODE>;
    const int nw = nch * bwd_splits(nch);
    return nw * Cfg::B * Cfg::ESP;
}

template <int L, typename XT, int MODE, int SG, bool CONC>
__device__ __forceinline__ void bwd_group(const int lb, const int n_dst, const int nslice, const int C,
                                          const int *__restrict__ row_ptr,
                                          const int *__restrict__ src, const float *__restrict__ vec,
                                          const XT *__restrict__ x, const float *__restrict__ w,
                                          const float *__restrict__ G, const float *__restrict__ ggx,
                                          const float *__restrict__ ggw, const float *__restrict__ ggvec,
                                          float *__restrict__ part, float *__restrict__ ow,
                                          float *__restrict__ ovec, const uint32_t flags, float *lds,
                                          float *__restrict__ grws, const int64_t n_edges)
{
    using Cfg = BwdCfg<L, MODE>;
    constexpr int B = Cfg::B, ES = Cfg::ES, NV = Cfg::NV, DSHP = Cfg::DSHP, PK = Cfg::PK;
    constexpr bool V2 = Cfg::V2;
    constexpr Groups GR = Cfg::GR;
    constexpr SrcGroupInfo GI = src_group_info(kTab<L>, GR, SG);
    constexpr int P = kTab<L>.P, DIN = kTab<L>.din_rows, DOUT = kTab<L>.dout_rows, DSH = kTab<L>.dsh;
    constexpr int NP = GI.np, NXR = GI.nxr, NGR = GI.ngr;
    constexpr int BLO = sh_lo(kTab<L>, GI.p0, GI.p1), BHI = sh_hi(kTab<L>, GI.p0, GI.p1);
    constexpr int L1A = kTab<L>.path[GI.p0].l1;
    constexpr int SHARED_ROWS = GI.shares_first_l1 ? 2 * L1A + 1 : 0;  // part rows an earlier group began

    const int lane = threadIdx.x & 63, wv = wave_id();
    const int nch = (C + 63) >> 6, nsp = bwd_splits(nch);
    const int ch = wv % nch, sp = wv / nch;  // channel chunk, edge split
    // workgroup = (destination node, slice of its in-edges): the in-edges
    // are independent given G[i], so long rows split over several workgroups
    // (more, shorter work units: no tail when there are few nodes)
    const int i = lb / nslice, sl = lb - i * nslice;
    if (i >= n_dst)
        return;
    const int u = ch * 64 + lane;
    const bool active = u < C;
    const uint32_t off4 = active ? static_cast<uint32_t>(u) * 4u : kOOB;
    const uint32_t offx = active ? static_cast<uint32_t>(u) * static_cast<uint32_t>(sizeof(XT)) : kOOB;
    const bool want_vec = ovec != nullptr, want_x = part != nullptr;
    // where this group's gr / dr go: in sequence (CONC false) later groups add
    // to the earlier groups' result in ovec; side by side (CONC true) group 0
    // writes ovec and group g > 0 its own slice of grws, added in group order
    // afterwards
    float *const gdst = (CONC && SG > 0) ? grws + static_cast<int64_t>(SG - 1) * 3 * n_edges : ovec;
    constexpr bool GADD = !CONC && SG > 0;
    const bool has_xp = V2 && ggx != nullptr, has_wp = V2 && ggw != nullptr, has_rp = V2 && ggvec != nullptr;
    const uint32_t rowb = static_cast<uint32_t>(C) * 4u, rowx = static_cast<uint32_t>(C) * sizeof(XT);

    // LDS: per wave the batch [B][ES] and two park slots [2][B][PK]
    const int nw = nch * nsp;
    float *blds = lds + wv * (B * ES);
    float *pall = lds + nw * (B * ES);
    float *plds = pall + wv * (2 * B * PK);

    const int rb = row_ptr[i], rlen = row_ptr[i + 1] - rb;
    const int s0 = rb + static_cast<int>(static_cast<int64_t>(rlen) * sl / nslice);
    const int s1 = rb + static_cast<int>(static_cast<int64_t>(rlen) * (sl + 1) / nslice);
    const int kbase = s0 + sp, len = s1 - s0;
    const int cnt = len > sp ? (len - sp + nsp - 1) / nsp : 0;
    const int nbatch = ((len + nsp - 1) / nsp + B - 1) / B;
    auto epos = [&](int t) { return kbase + t * nsp; };  // the split's t-th edge

    // node-resident G[i] rows of this group's paths
    float g[NGR];
    {
        const rsrc_t rg = make_rsrc(G + static_cast<int64_t>(i) * (DOUT * C), DOUT * C * 4u);
        static_range<0, NGR>([&](auto q) { g[q] = bload<float>(rg, off4, (GI.gr0 + q) * rowb); });
    }

    // Operands of one edge: the w (W') rows of the group's paths and the x
    // (X') rows of its l1 values. A path's weight row takes the next edge's
    // as soon as the path is done, an l1 block's x rows after the block's
    // last path of the group.
    struct Ops {
        float w[NP], wp[V2 ? NP : 1], x[NXR], xp[V2 ? NXR : 1];
    };
    struct EdgeRsrc {
        rsrc_t w, wp, x, xp;
    };
    auto edge_rsrc = [&](int e, bool valid) {
        const int j = src[e];
        EdgeRsrc r;
        r.w = make_rsrc(w + static_cast<int64_t>(e) * (P * C), valid ? P * C * 4u : 0u);
        r.x = make_rsrc(x + static_cast<int64_t>(j) * (DIN * C), valid ? DIN * C * static_cast<uint32_t>(sizeof(XT)) : 0u);
        r.wp = make_rsrc(has_wp ? ggw + static_cast<int64_t>(e) * (P * C) : nullptr, has_wp && valid ? P * C * 4u : 0u);
        r.xp = make_rsrc(has_xp ? ggx + static_cast<int64_t>(j) * (DIN * C) : nullptr, has_xp && valid ? DIN * C * 4u : 0u);
        return r;
    };
    Ops o;
    auto load_w = [&](auto p, const EdgeRsrc &r) {
        constexpr int WQ = p - GI.p0;
        o.w[WQ] = bload<float, kNT>(r.w, off4, p * rowb);
        if constexpr (V2)
            o.wp[WQ] = bload<float, kNT>(r.wp, off4, p * rowb);
    };
    auto load_x = [&](auto q, const EdgeRsrc &r) {  // q: x row within the group
        o.x[q] = bload_x<float, XT>(r.x, offx, (GI.xr0 + q) * rowx);
        if constexpr (V2)
            o.xp[q] = bload<float>(r.xp, off4, (GI.xr0 + q) * rowb);
    };
    auto load_all = [&](const EdgeRsrc &r) {
        static_range<GI.p0, GI.p1>([&](auto p) { load_w(p, r); });
        static_range<0, NXR>([&](auto q) { load_x(q, r); });
    };

    // Per batch, lane = edge: Y (, Yd) and the coefficients of the gr / dr
    // contraction.
    auto prologue = [&](int t0, int nb) {
        wave_sync_lds();
        if (lane < nb) {
            const int e = epos(t0 + lane);
            const float rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
            float *ep = blds + lane * ES;
            float4 *cp = reinterpret_cast<float4 *>(ep + NV * DSHP);
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
            }
        }
        wave_sync_lds();
    };

    // gr / dr of a finished batch from the parked per-chunk sums (several
    // chunks only): lane = edge, chunk 0's wave of the split adds the chunks
    // in order; the park slots alternate by batch.
    auto epilogue = [&](int t0, int nb, int slot) {
        __syncthreads();
        if (want_vec && ch == 0 && lane < nb) {
            float g0 = 0.f, g1 = 0.f, g2 = 0.f;
            for (int c = 0; c < nch; ++c) {
                const float *pp = pall + (sp * nch + c) * (2 * B * PK) + (slot * B + lane) * PK;
                g0 += pp[0];
                g1 += pp[1];
                g2 += pp[2];
            }
            float *gp = gdst + 3 * static_cast<int64_t>(epos(t0 + lane));
            if (GADD) {
                g0 += gp[0];
                g1 += gp[1];
                g2 += gp[2];
            }
            gp[0] = g0;
            gp[1] = g1;
            gp[2] = g2;
        }
    };

    float Z[DSH], Z2[V2 ? DSH : 1];
    static_range<0, DSH>([&](auto b) {
        Z[b] = 0.f;
        if constexpr (V2)
            Z2[b] = 0.f;
    });

    // One edge, path by path: K from the resident G rows, the part sums of
    // the edge's l1 blocks (stored when a block is done), the weight
    // cotangent (stored) and the Z sums.
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
        const rsrc_t rpt = make_rsrc(want_x ? part + static_cast<int64_t>(e) * (DIN * C) : nullptr,
                                     want_x ? DIN * C * 4u : 0u);
        float acc[NXR];  // the edge's part rows of the group's l1 blocks
        // VJP-of-VJP per path in the order that needs one FMA fewer per
        // (m1, m2) group: with K[a, b] = sum_c C g[c] and, per m2 = b,
        //   u[b] = sum_a X'[a] K,  v[b] = sum_a x[a] K,  eta[b] = W' Y_b + w Yd_b,
        // the part rows take part[a] += eta[b] K per group, and
        //   dw = sum_b Y_b u[b] + Yd_b v[b],  Z[b] += w u[b] + W' v[b],  Z2[b] += w v[b]
        // per (path, b): the same sums as s, sd, xx, wx below, regrouped.
        auto path_uv = [&](auto p) {
            constexpr Path pa = kTab<L>.path[p];
            constexpr int d1 = 2 * pa.l1 + 1, d2 = 2 * pa.l2 + 1, YB = pa.y_row;
            constexpr int XO = pa.x_row - GI.xr0, GO = pa.out_row - GI.gr0, WQ = p - GI.p0;
            constexpr int PA0 = kTab<L>.path_ab0[p], PA1 = kTab<L>.path_ab0[p + 1];
            constexpr bool FIRST_OF_L1 = p == GI.p0 || !same_l1(kTab<L>, p - 1, p);
            constexpr bool LAST_OF_L1 = p + 1 == GI.p1 || !same_l1(kTab<L>, p, p + 1);
            const float wv_ = o.w[WQ], wpp = o.wp[WQ];
            float eta[d2], u[d2], v[d2];
            static_range<0, d2>([&](auto m) {
                if constexpr (ab_touches_b(kTab<L>, PA0, PA1, YB + m))
                    eta[m] = fmaf(wv_, Ydb[YB + m], wpp * Yb[YB + m]);
            });
            static_range<PA0, PA1>([&](auto gq) {
                constexpr ABGroup ag = kTab<L>.ab[gq];
                constexpr int a = ag.m1 + pa.l1, m = pa.l2 + ag.m2;
                float K;
                static_range<ag.t0, ag.t1>([&](auto ti) {
                    constexpr Entry en = kTab<L>.nz[kTab<L>.ab_entries[ti]];
                    if constexpr (ti == ag.t0)
                        K = en.fval * g[GO + en.m3 + pa.l3];
                    else
                        K = fmaf(en.fval, g[GO + en.m3 + pa.l3], K);
                });
                if constexpr (ab_first_b(kTab<L>, PA0, gq)) {
                    u[m] = o.xp[XO + a] * K;
                    v[m] = o.x[XO + a] * K;
                } else {
                    u[m] = fmaf(o.xp[XO + a], K, u[m]);
                    v[m] = fmaf(o.x[XO + a], K, v[m]);
                }
                if constexpr (FIRST_OF_L1 && ab_first_m1(kTab<L>, gq))
                    acc[XO + a] = eta[m] * K;
                else
                    acc[XO + a] = fmaf(eta[m], K, acc[XO + a]);
            });
            // the path's weight row takes the next edge's
            load_w(p, nx);
            float gwv = 0.f;
            bool started = false;
            static_range<0, d2>([&](auto m) {
                constexpr int b = YB + m;
                if constexpr (ab_touches_b(kTab<L>, PA0, PA1, b)) {
                    gwv = started ? fmaf(Yb[b], u[m], fmaf(Ydb[b], v[m], gwv)) : fmaf(Yb[b], u[m], Ydb[b] * v[m]);
                    started = true;
                    if constexpr (!ab_touches_b(kTab<L>, GI.ab0, PA0, b)) {  // b's first path in the group
                        Z[b] = fmaf(wv_, u[m], wpp * v[m]);
                        Z2[b] = wv_ * v[m];
                    } else {
                        Z[b] = fmaf(wv_, u[m], fmaf(wpp, v[m], Z[b]));
                        Z2[b] = fmaf(wv_, v[m], Z2[b]);
                    }
                }
            });
            bstore<float, kNT>(gwv, rgw, off4, p * rowb);
            if constexpr (LAST_OF_L1) {
                static_range<0, d1>([&](auto a) {
                    constexpr int r = XO + a;
                    float val = acc[r];
                    if constexpr (r < SHARED_ROWS)
                        val += bload<float>(rpt, off4, (GI.xr0 + r) * rowb);
                    bstore<float, kNT>(val, rpt, off4, (GI.xr0 + r) * rowb);
                });
                static_range<0, d1>([&](auto a) { load_x(ic<XO + a>{}, nx); });
            }
        };
        static_range<GI.p0, GI.p1>([&](auto p) {
            if constexpr (V2 && ETP_BWD_UV && uv_cheaper(kTab<L>, p)) {
                path_uv(p);
                return;
            }
            constexpr Path pa = kTab<L>.path[p];
            constexpr int d1 = 2 * pa.l1 + 1;
            constexpr int XO = pa.x_row - GI.xr0, GO = pa.out_row - GI.gr0, WQ = p - GI.p0;
            constexpr bool FIRST_OF_L1 = p == GI.p0 || !same_l1(kTab<L>, p - 1, p);
            constexpr bool LAST_OF_L1 = p + 1 == GI.p1 || !same_l1(kTab<L>, p, p + 1);
            const float wv_ = o.w[WQ];
            float wpp = 0.f;
            if constexpr (V2)
                wpp = o.wp[WQ];
            float wx[d1], xx[V2 ? d1 : 1], s[d1], sd[V2 ? d1 : 1];
            static_range<0, d1>([&](auto a) {
                wx[a] = wv_ * o.x[XO + a];
                if constexpr (V2)
                    xx[a] = fmaf(wv_, o.xp[XO + a], wpp * o.x[XO + a]);
            });
            static_range<kTab<L>.path_ab0[p], kTab<L>.path_ab0[p + 1]>([&](auto gq) {
                constexpr ABGroup ag = kTab<L>.ab[gq];
                constexpr int a = ag.m1 + pa.l1, b = pa.y_row + pa.l2 + ag.m2;
                float K;
                static_range<ag.t0, ag.t1>([&](auto ti) {
                    constexpr Entry en = kTab<L>.nz[kTab<L>.ab_entries[ti]];
                    if constexpr (ti == ag.t0)
                        K = en.fval * g[GO + en.m3 + pa.l3];
                    else
                        K = fmaf(en.fval, g[GO + en.m3 + pa.l3], K);
                });
                if constexpr (ab_first_m1(kTab<L>, gq)) {
                    s[a] = Yb[b] * K;
                    if constexpr (V2)
                        sd[a] = Ydb[b] * K;
                } else {
                    s[a] = fmaf(Yb[b], K, s[a]);
                    if constexpr (V2)
                        sd[a] = fmaf(Ydb[b], K, sd[a]);
                }
                if constexpr (ab_first_b(kTab<L>, GI.ab0, gq)) {
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
            // the path's weight row takes the next edge's
            load_w(p, nx);
            float gwv;
            static_range<0, d1>([&](auto a) {
                float pv;
                if constexpr (!V2)
                    pv = wv_ * s[a];
                else
                    pv = fmaf(wpp, s[a], wv_ * sd[a]);
                if constexpr (FIRST_OF_L1)
                    acc[XO + a] = pv;
                else
                    acc[XO + a] += pv;
                if constexpr (!V2) {
                    if constexpr (a == 0)
                        gwv = o.x[XO + a] * s[a];
                    else
                        gwv = fmaf(o.x[XO + a], s[a], gwv);
                } else {
                    if constexpr (a == 0)
                        gwv = fmaf(o.xp[XO + a], s[a], o.x[XO + a] * sd[a]);
                    else
                        gwv = fmaf(o.xp[XO + a], s[a], fmaf(o.x[XO + a], sd[a], gwv));
                }
            });
            bstore<float, kNT>(gwv, rgw, off4, p * rowb);
            if constexpr (LAST_OF_L1) {
                // the l1 block is done for this edge: its part rows are
                // stored (added to an earlier group's where the block began
                // there) and its x rows take the next edge's
                static_range<0, d1>([&](auto a) {
                    constexpr int r = XO + a;
                    float v = acc[r];
                    if constexpr (r < SHARED_ROWS)
                        v += bload<float>(rpt, off4, (GI.xr0 + r) * rowb);
                    bstore<float, kNT>(v, rpt, off4, (GI.xr0 + r) * rowb);
                });
                static_range<0, d1>([&](auto a) { load_x(ic<XO + a>{}, nx); });
            }
        });
    };

    // The edge's gr / dr partial over this wave's channels: Z contracted
    // with the edge's coefficients per lane, then a fixed-order DPP sum of
    // the three components (exact in lane 63).
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
    };

    int kb = 0, done = 0;
    static_range<0, NGR>([&](auto q) { settle(g[q]); });
    for (int t = 0; t < cnt; ++t) {
        const int batch0 = t - kb, nb = min(B, cnt - batch0), e = epos(t);
        if (kb == 0) {
            prologue(t, nb);
            load_all(edge_rsrc(e, true));
        }
        const bool more = kb + 1 < nb;
        const EdgeRsrc nx = edge_rsrc(more ? e + nsp : e, more);
        const float *ep = blds + kb * ES;
        compute(ep, e, nx);
        float g0, g1, g2;
        fold(ep, g0, g1, g2);
        if (want_vec) {
            if (nch == 1) {
                if (lane == 63) {
                    float *gp = gdst + 3 * static_cast<int64_t>(e);
                    if (GADD) {
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
        if (++kb == nb) {
            if (nch > 1)
                epilogue(batch0, nb, done & 1);
            kb = 0;
            ++done;
        }
    }
    if (nch > 1)
        for (; done < nbatch; ++done)
            epilogue(cnt, 0, done & 1);

}

template <int L, typename XT, int MODE, int SG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BwdCfg<L, MODE>::WPE)))
    bwd_kernel(const int n_dst, const int nslice, const int C, const int *__restrict__ row_ptr, const int *__restrict__ src,
               const float *__restrict__ vec, const XT *__restrict__ x, const float *__restrict__ w,
               const float *__restrict__ G, const float *__restrict__ ggx, const float *__restrict__ ggw,
               const float *__restrict__ ggvec, float *__restrict__ part, float *__restrict__ ow,
               float *__restrict__ ovec, const uint32_t flags)
{
    extern __shared__ float lds[];
    bwd_group<L, XT, MODE, SG, false>(xcd_remap(blockIdx.x, gridDim.x), n_dst, nslice, C, row_ptr, src, vec, x, w, G,
                                      ggx, ggw, ggvec, part, ow, ovec, flags, lds, nullptr, 0);
}

// Every path group in one launch: one flat grid over (node, in-edge slice,
// group) with the group varying fastest, so that a node's groups run side by
// side on one XCD (sharing its edges' indices, bond vectors and x rows in L2)
// and groups bound by arithmetic overlap with groups bound by memory. Only
// for tables whose groups write disjoint part rows; gr / dr partials of the
// groups after the first go to grws.
template <int L, typename XT, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BwdCfg<L, MODE>::WPE)))
    bwd_kernel_all(const int n_dst, const int nslice, const int C, const int *__restrict__ row_ptr,
                   const int *__restrict__ src, const float *__restrict__ vec, const XT *__restrict__ x,
                   const float *__restrict__ w, const float *__restrict__ G, const float *__restrict__ ggx,
                   const float *__restrict__ ggw, const float *__restrict__ ggvec, float *__restrict__ part,
                   float *__restrict__ ow, float *__restrict__ ovec, const uint32_t flags, float *__restrict__ grws,
                   const int64_t n_edges)
{
    extern __shared__ float lds[];
    constexpr Groups GR = BwdCfg<L, MODE>::GR;
    const int flat = xcd_remap(blockIdx.x, gridDim.x);
    const int g = flat % GR.n, lb = flat / GR.n;
    static_range<0, GR.n>([&](auto SG) __attribute__((always_inline)) {
        if (g == SG)
            bwd_group<L, XT, MODE, SG, true>(lb, n_dst, nslice, C, row_ptr, src, vec, x, w, G, ggx, ggw, ggvec, part,
                                             ow, ovec, flags, lds, grws, n_edges);
    });
}

// gr += the partials of groups 1 .. NX (in group order), per edge.
template <int NX>
__global__ void __launch_bounds__(256) bwd_gr_sum_kernel(const int64_t n3, const float *__restrict__ grws,
                                                         float *__restrict__ ovec)
{
    for (int64_t t = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; t < n3;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        float v = ovec[t];
#pragma unroll
        for (int k = 0; k < NX; ++k)
            v += grws[k * n3 + t];
        ovec[t] = v;
    }
}

// Whether the path groups of a table write disjoint part rows (each l1
// block inside one group), so that they may run side by side.
template <int L, int MODE>
constexpr bool bwd_groups_disjoint()
{
    constexpr Groups GR = BwdCfg<L, MODE>::GR;
    for (int k = 1; k < GR.n; ++k)
        if (GR.p0[k] > 0 && kTab<L>.path[GR.p0[k] - 1].l1 == kTab<L>.path[GR.p0[k]].l1)
            return false;
    return true;
}

// gx[j] (+)= sum over j's out-edges, in the order of the stable transpose, of
// the per-edge part rows (each a contiguous block of n floats, n = Din C):
// thread t owns V consecutive floats of one node's block (t over n_src * n / V,
// so the threads of one node read one edge's block together), and adds its
// node's edges one after another in transpose order.
template <int V>
__global__ void __launch_bounds__(256) bwd_gather_kernel(const int64_t total, const int per,
                                                         const int *__restrict__ src_ptr,
                                                         const int *__restrict__ perm, const float *__restrict__ part,
                                                         float *__restrict__ gx, const uint32_t flags)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    using VT = std::conditional_t<V == 4, f32x4, float>;
    const VT *pv = reinterpret_cast<const VT *>(part);
    for (int64_t t = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; t < total;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t j = t / per;
        const int q = static_cast<int>(t - j * per);
        const int k0 = src_ptr[j], k1 = src_ptr[j + 1];
        VT s = VT(0.f);
        int k = k0;
        for (; k + 4 <= k1; k += 4) {
            const int e0 = perm[k], e1 = perm[k + 1], e2 = perm[k + 2], e3 = perm[k + 3];
            const VT a = __builtin_nontemporal_load(pv + static_cast<int64_t>(e0) * per + q);
            const VT b = __builtin_nontemporal_load(pv + static_cast<int64_t>(e1) * per + q);
            const VT c = __builtin_nontemporal_load(pv + static_cast<int64_t>(e2) * per + q);
            const VT d = __builtin_nontemporal_load(pv + static_cast<int64_t>(e3) * per + q);
            s += a;  // (element-wise; one edge after another)
            s += b;
            s += c;
            s += d;
        }
        for (; k < k1; ++k)
            s += __builtin_nontemporal_load(pv + static_cast<int64_t>(perm[k]) * per + q);
        VT *o = reinterpret_cast<VT *>(gx) + t;
        if (flags & 1u)
            s += *o;
        *o = s;
    }
}

template <int L, typename XT, int MODE>
static hipError_t launch_bwd_t(const ConvArgs &a, float *part, int64_t E, float *grws)
{
    using Cfg = BwdCfg<L, MODE>;
    constexpr Groups GR = Cfg::GR;
    const int nch = (a.C + 63) / 64;
    const size_t lds_bytes = sizeof(float) * bwd_lds_floats<L, MODE>(nch);
    hipError_t err = hipSuccess;
    if (a.n_dst > 0 && (part || a.ow || a.ovec)) {
        // in-edge slices per node: enough workgroups to fill the chip a few
        // times over, at least 16 edges per slice on average
        int nslice = static_cast<int>((4096 + a.n_dst - 1) / a.n_dst);
        const int64_t by_deg = E / (16 * static_cast<int64_t>(a.n_dst));
        nslice = static_cast<int>(nslice < by_deg ? nslice : by_deg);
        nslice = nslice < 1 ? 1 : (nslice > 16 ? 16 : nslice);
        if (static_cast<int64_t>(a.n_dst) * nslice * GR.n > 0x7FFFFFFF)
            return hipErrorInvalidValue;
        constexpr bool side_by_side = GR.n > 1 && GR.n - 1 <= kBwdGrSlices && bwd_groups_disjoint<L, MODE>();
        bool one_launch = false;
        if constexpr (side_by_side) {
            one_launch = grws || !a.ovec;  // gr partials need their slices
            if (one_launch) {
                const int64_t nb = static_cast<int64_t>(a.n_dst) * nslice * GR.n;
                hipLaunchKernelGGL((bwd_kernel_all<L, XT, MODE>), dim3(static_cast<unsigned>(nb)),
                                   dim3(64 * nch * bwd_splits(nch)), lds_bytes, a.stream, a.n_dst, nslice, a.C,
                                   a.row_ptr, a.src, a.vec, static_cast<const XT *>(a.x), a.w, a.G, a.ggx, a.ggw,
                                   a.ggvec, part, a.ow, a.ovec, a.flags, grws, E);
                err = hipGetLastError();
                if (err == hipSuccess && a.ovec && E > 0) {
                    const int64_t n3 = 3 * E, blocks = (n3 + 255) / 256;
                    hipLaunchKernelGGL((bwd_gr_sum_kernel<GR.n - 1>),
                                       dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)), dim3(256), 0,
                                       a.stream, n3, grws, a.ovec);
                    err = hipGetLastError();
                }
            }
        }
        if (!one_launch) {
            // one launch per path group, in order: later groups add to gr / dr
            // and to the part rows of an l1 block an earlier group began
            static_range<0, GR.n>([&](auto g) {
                if (err != hipSuccess)
                    return;
                hipLaunchKernelGGL((bwd_kernel<L, XT, MODE, g>), dim3(a.n_dst * nslice),
                                   dim3(64 * nch * bwd_splits(nch)), lds_bytes, a.stream, a.n_dst, nslice, a.C,
                                   a.row_ptr, a.src, a.vec, static_cast<const XT *>(a.x), a.w, a.G, a.ggx, a.ggw,
                                   a.ggvec, part, a.ow, a.ovec, a.flags);
                err = hipGetLastError();
            });
        }
    }
    if (err != hipSuccess || !a.ox || a.n_src == 0)
        return err;
    // the node gradient: the part rows summed per source in transpose order
    const int n = kTab<L>.din_rows * a.C;
    const int V = n % 4 == 0 ? 4 : 1;
    const int64_t total = static_cast<int64_t>(a.n_src) * (n / V);
    const int64_t blocks = (total + 255) / 256;
    const unsigned grid = static_cast<unsigned>(blocks < (1 << 20) ? blocks : (1 << 20));
    if (V == 4)
        hipLaunchKernelGGL(bwd_gather_kernel<4>, dim3(grid), dim3(256), 0, a.stream, total, n / 4, a.src_ptr, a.perm,
                           part, a.ox, a.flags);
    else
        hipLaunchKernelGGL(bwd_gather_kernel<1>, dim3(grid), dim3(256), 0, a.stream, total, n, a.src_ptr, a.perm,
                           part, a.ox, a.flags);
    return hipGetLastError();
}

#if !defined(ETP_L) || !defined(ETP_XT) || !defined(ETP_MODE)
#error "compile this file once per (l_max, dtype, mode) with -DETP_L=0..4 -DETP_XT=0|1 -DETP_MODE=0|1"
#endif

hipError_t ETP_RUN_NAME(bwd, ETP_L, ETP_XT, ETP_MODE)(const ConvArgs &a, float *part, int64_t n_edges, float *grws)
{
    using XT = std::conditional_t<ETP_XT == 1, bf16raw, float>;
    return launch_bwd_t<ETP_L, XT, ETP_MODE>(a, part, n_edges, grws);
}

}  // namespace etp
