// etp_edge_tp.hip -- the edge-local tensor product: the convolution's
// message without the destination sum, one output block per edge (the
// pair-wise tensor product of Allegro, whose energy is a sum of per-pair
// terms: "Scaling the leading accuracy of deep equivariant models to
// biomolecular simulations of realistic size", section "Proposed method").
//
//   out[e, off_p + m3, u] = w[e, p, u] sum_{(m1, m2, m3) in p} C Y_{l2 m2}(r_e) V[e, l1 m1, u]
//
// and its VJP (gV, gw and the bond-vector gradient gr).
//
// Mapping (gfx950, wave64): lane = channel. The forward gives each wave a
// run of consecutive edges of one 64-channel chunk; per edge the SH (the
// same for every lane) and, per (m1, m3) pair of a path, the coefficient
// K = sum_{m2} C Y_{m2} are formed in registers, then one FMA per pair and
// lane. The VJP gives each wave whole edges (every channel chunk), so the
// per-edge sums over channels that build gr stay in registers until one
// fixed-order DPP reduction per SH component. Streamed rows (V, w, G, out,
// gV, gw) go through buffer descriptors with non-temporal hints; lanes past C
// use an out-of-range offset, so their loads return 0 and their stores drop.
// No atomics anywhere: results are bitwise deterministic.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "etp_device.hpp"
#include "etp_tables.hpp"

namespace etp {

constexpr int kEdgeTpRun = 8;  // edges per wave in the forward

// Coefficient of the (m1, m3) pair q of a path: sum over its entries of C Y[l2, m2].
template <int L, int Q>
__device__ __forceinline__ float pair_coef(const float *Y)
{
    constexpr Pair pr = kTab<L>.pair[Q];
    constexpr Path pa = kTab<L>.path[pr.path];
    float k = 0.f;
    static_range<pr.t0, pr.t1>([&](auto tc) {
        constexpr Entry e = kTab<L>.nz[kTab<L>.pair_entries[tc]];
        k = __builtin_fmaf(e.fval, Y[pa.y_row + pa.l2 + e.m2], k);
    });
    return k;
}

template <int L, bool ACC>
__global__ void __launch_bounds__(256) edge_tp_fwd_kernel(const int64_t E, const int C, const float *__restrict__ vec,
                                                          const float *__restrict__ V, const float *__restrict__ w,
                                                          float *__restrict__ out)
{
    constexpr int P = kTab<L>.P, DIN = kTab<L>.din_rows, DOUT = kTab<L>.dout_rows, DSH = kTab<L>.dsh;
    const int lane = threadIdx.x & 63;
    const int cw = (C + 63) >> 6;
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
    const int chunk = static_cast<int>(gw % cw);
    const int64_t e0 = (gw / cw) * kEdgeTpRun;
    if (e0 >= E)
        return;
    const int u = chunk * 64 + lane;
    const uint32_t vo = u < C ? static_cast<uint32_t>(u) * 4u : kOOB;
    const uint32_t rowb = static_cast<uint32_t>(C) * 4u;
    const int64_t e1 = e0 + kEdgeTpRun < E ? e0 + kEdgeTpRun : E;
    uint32_t rb = rowb;
    for (int64_t e = e0; e < e1; ++e) {
        // an opaque copy of the row stride per edge, so that the per-row
        // offsets are formed next to their loads instead of being hoisted
        // out of the loop as dozens of live scalars
        asm volatile("" : "+s"(rb));
        const uint32_t rowb = rb;
        const rsrc_t rv = make_rsrc(V + e * DIN * C, DIN * rowb);
        const rsrc_t rw = make_rsrc(w + e * P * C, P * rowb);
        const rsrc_t ro = make_rsrc(out + e * DOUT * C, DOUT * rowb);
        float x[DIN];
        static_range<0, DIN>([&](auto r) { x[r] = bload<float, kNT>(rv, vo, r * rowb); });
        float Y[DSH];
        sh_value<L>(vec[3 * e], vec[3 * e + 1], vec[3 * e + 2], Y);
        static_range<0, P>([&](auto pc) {
            constexpr Path pa = kTab<L>.path[pc];
            const float wp = bload<float, kNT>(rw, vo, pc * rowb);
            float acc[2 * pa.l3 + 1];
            static_range<0, 2 * pa.l3 + 1>([&](auto m) { acc[m] = 0.f; });
            static_range<pa.pr0, pa.pr1>([&](auto qc) {
                constexpr Pair pr = kTab<L>.pair[qc];
                const float k = pair_coef<L, qc>(Y);
                acc[pr.m3 + pa.l3] = __builtin_fmaf(k, x[pa.x_row + pa.l1 + pr.m1], acc[pr.m3 + pa.l3]);
            });
            static_range<0, 2 * pa.l3 + 1>([&](auto m) {
                const uint32_t so = (pa.out_row + m) * rowb;
                float v = wp * acc[m];
                if constexpr (ACC)
                    v += bload<float>(ro, vo, so);
                bstore<float, kNT>(v, ro, vo, so);
            });
        });
    }
}

// VJP: one wave per edge, every channel chunk; gr needs the sum over all
// channels. A null gV or gw gets an empty buffer range (its stores drop), so
// the loops carry no branches: branches inside the unrolled path loop split
// the compiler's scheduling regions and tripled the register count.
template <int L, bool ACC>
__global__ void __launch_bounds__(256) edge_tp_vjp_kernel(const int64_t E, const int C, const float *__restrict__ vec,
                                                          const float *__restrict__ V, const float *__restrict__ w,
                                                          const float *__restrict__ G, float *__restrict__ gV,
                                                          float *__restrict__ gwt, float *__restrict__ gr)
{
    constexpr int P = kTab<L>.P, DIN = kTab<L>.din_rows, DOUT = kTab<L>.dout_rows, DSH = kTab<L>.dsh;
    const int lane = threadIdx.x & 63;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
    if (e >= E)
        return;
    const int cw = (C + 63) >> 6;
    const uint32_t rowb = static_cast<uint32_t>(C) * 4u;
    const rsrc_t rv = make_rsrc(V + e * DIN * C, DIN * rowb);
    const rsrc_t rw = make_rsrc(w + e * P * C, P * rowb);
    const rsrc_t rg = make_rsrc(G + e * DOUT * C, DOUT * rowb);
    const rsrc_t rgv = make_rsrc(gV ? gV + e * DIN * C : nullptr, gV ? DIN * rowb : 0u);
    const rsrc_t rgw = make_rsrc(gwt ? gwt + e * P * C : nullptr, gwt ? P * rowb : 0u);

    D3 Yd[DSH];
    sh_grad<L>(vec[3 * e], vec[3 * e + 1], vec[3 * e + 2], Yd);
    float Y[DSH];
    static_range<0, DSH>([&](auto b) { Y[b] = Yd[b].v; });
    float Z[DSH];  // this lane's share of dL/dY
    static_range<0, DSH>([&](auto b) { Z[b] = 0.f; });

    for (int chunk = 0; chunk < cw; ++chunk) {
        // opaque Y per chunk: the pair coefficients are recomputed next to
        // their use instead of being hoisted out of the chunk loop
        static_range<0, DSH>([&](auto b) { settle(Y[b]); });
        const int u = chunk * 64 + lane;
        const uint32_t vo = u < C ? static_cast<uint32_t>(u) * 4u : kOOB;
        float x[DIN], gx[DIN];
        static_range<0, DIN>([&](auto r) {
            x[r] = bload<float, kNT>(rv, vo, r * rowb);
            gx[r] = 0.f;
        });
        // the next path's G rows and weight load while the current path
        // computes (two slots of 2 l_max + 1 rows)
        float gb[2][2 * L + 1], wb[2];
        auto fetch = [&](auto pc, auto slot) {
            constexpr Path pa = kTab<L>.path[pc];
            wb[slot] = bload<float, kNT>(rw, vo, pc * rowb);
            static_range<0, 2 * pa.l3 + 1>(
                [&](auto m) { gb[slot][m] = bload<float, kNT>(rg, vo, (pa.out_row + m) * rowb); });
        };
        fetch(ic<0>{}, ic<0>{});
        static_range<0, P>([&](auto pc) {
            constexpr Path pa = kTab<L>.path[pc];
            constexpr int cur = pc % 2;
            if constexpr (pc + 1 < P)
                fetch(ic<pc + 1>{}, ic<1 - cur>{});
            const float wp = wb[cur];
            float s = 0.f;  // dL/dw[e, p, u]
            static_range<pa.pr0, pa.pr1>([&](auto qc) {
                constexpr Pair pr = kTab<L>.pair[qc];
                const float xm = x[pa.x_row + pa.l1 + pr.m1], gm = gb[cur][pr.m3 + pa.l3];
                const float k = pair_coef<L, qc>(Y);
                const float t = xm * gm;
                s = __builtin_fmaf(k, t, s);
                gx[pa.x_row + pa.l1 + pr.m1] = __builtin_fmaf(wp * k, gm, gx[pa.x_row + pa.l1 + pr.m1]);
                const float wt = wp * t;
                static_range<pr.t0, pr.t1>([&](auto tc) {
                    constexpr Entry en = kTab<L>.nz[kTab<L>.pair_entries[tc]];
                    Z[pa.y_row + pa.l2 + en.m2] = __builtin_fmaf(en.fval, wt, Z[pa.y_row + pa.l2 + en.m2]);
                });
            });
            {
                float v = s;
                if constexpr (ACC)
                    v += bload<float>(rgw, vo, pc * rowb);
                bstore<float, kNT>(v, rgw, vo, pc * rowb);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        static_range<0, DIN>([&](auto r) {
            float v = gx[r];
            if constexpr (ACC)
                v += bload<float>(rgv, vo, r * rowb);
            bstore<float, kNT>(v, rgv, vo, r * rowb);
        });
    }
    if (gr) {
        // gr = sum_b (sum over channels of Z_b) dY_b/dr, reduced in fixed order
        float g0 = 0.f, g1 = 0.f, g2 = 0.f;
        static_range<0, DSH>([&](auto b) {
            const float zb = wave_sum_to_lane63(Z[b]);
            g0 = __builtin_fmaf(zb, Yd[b].g0, g0);
            g1 = __builtin_fmaf(zb, Yd[b].g1, g1);
            g2 = __builtin_fmaf(zb, Yd[b].g2, g2);
        });
        if (lane == 63) {
            float *ge = gr + 3 * e;
            if constexpr (ACC) {
                g0 += ge[0];
                g1 += ge[1];
                g2 += ge[2];
            }
            ge[0] = g0;
            ge[1] = g1;
            ge[2] = g2;
        }
    }
}

// VJP of the VJP: with cotangents (V', W', R') on (gV, gw, gr), the
// gradients of S = <V', gV> + <W', gw> + <R', gr> with respect to V (dV), w
// (dw), vec (dr) and G (dG). With Yd = grad Y . R' and, per (m1, m3) pair,
// K = sum_{m2} C Y_{m2}, Kd = sum_{m2} C Yd_{m2}:
//   dG[p, m3] += K (w V'[m1] + W' V[m1]) + Kd w V[m1]
//   dV[m1]    += G[p, m3] (W' K + w Kd)
//   dw[p]     += G[p, m3] (K V'[m1] + Kd V[m1])
//   Z1[m2]    += C G (w V' + W' V),  Z2[m2] += C G w V
//   dr = sum_b (sum over channels of Z1_b) grad Y_b + (sum of Z2_b) H_b R'.
// One wave per edge, every channel chunk (as the VJP); the SH jets for dr are
// formed once more at the end instead of being held through the loop.
template <int L, bool ACC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(L <= 2 ? 4 : (L == 3 ? 2 : 1))))
edge_tp_vjp2_kernel(const int64_t E, const int C, const float *__restrict__ vec, const float *__restrict__ V,
                    const float *__restrict__ w, const float *__restrict__ G, const float *__restrict__ ggV,
                    const float *__restrict__ ggw, const float *__restrict__ ggvec, float *__restrict__ dV,
                    float *__restrict__ dw, float *__restrict__ dr, float *__restrict__ dG)
{
    constexpr int P = kTab<L>.P, DIN = kTab<L>.din_rows, DOUT = kTab<L>.dout_rows, DSH = kTab<L>.dsh;
    const int lane = threadIdx.x & 63;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
    if (e >= E)
        return;
    const int cw = (C + 63) >> 6;
    const uint32_t rowb = static_cast<uint32_t>(C) * 4u;
    // a null array is an empty range: its loads read 0 and its stores drop
    auto blk = [&](const float *base, int rows) {
        return make_rsrc(base ? base + e * rows * C : nullptr, base ? rows * rowb : 0u);
    };
    const rsrc_t rv = blk(V, DIN), rvp = blk(ggV, DIN), rw = blk(w, P), rwp = blk(ggw, P), rg = blk(G, DOUT);
    const rsrc_t rdv = blk(dV, DIN), rdw = blk(dw, P), rdg = blk(dG, DOUT);

    const float rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
    float px = 0.f, py = 0.f, pz = 0.f;
    if (ggvec) {
        px = ggvec[3 * e];
        py = ggvec[3 * e + 1];
        pz = ggvec[3 * e + 2];
    }
    float Y[DSH], Yd[DSH];
    sh_grad_emit<L>(rx, ry, rz, [&](auto b, const D3 &y) {
        Y[b] = y.v;
        Yd[b] = y.g0 * px + y.g1 * py + y.g2 * pz;
    });
    float Z1[DSH], Z2[DSH];
    static_range<0, DSH>([&](auto b) {
        Z1[b] = 0.f;
        Z2[b] = 0.f;
    });

    for (int chunk = 0; chunk < cw; ++chunk) {
        static_range<0, DSH>([&](auto b) {
            settle(Y[b]);
            settle(Yd[b]);
        });
        const int u = chunk * 64 + lane;
        const uint32_t vo = u < C ? static_cast<uint32_t>(u) * 4u : kOOB;
        float x[DIN], xp[DIN], gx[DIN];
        static_range<0, DIN>([&](auto r) {
            x[r] = bload<float, kNT>(rv, vo, r * rowb);
            xp[r] = bload<float, kNT>(rvp, vo, r * rowb);
            gx[r] = 0.f;
        });
        float gb[2][2 * L + 1], wb[2], wpb[2];
        auto fetch = [&](auto pc, auto slot) {
            constexpr Path pa = kTab<L>.path[pc];
            wb[slot] = bload<float, kNT>(rw, vo, pc * rowb);
            wpb[slot] = bload<float, kNT>(rwp, vo, pc * rowb);
            static_range<0, 2 * pa.l3 + 1>(
                [&](auto m) { gb[slot][m] = bload<float, kNT>(rg, vo, (pa.out_row + m) * rowb); });
        };
        fetch(ic<0>{}, ic<0>{});
        static_range<0, P>([&](auto pc) {
            constexpr Path pa = kTab<L>.path[pc];
            constexpr int cur = pc % 2;
            if constexpr (pc + 1 < P)
                fetch(ic<pc + 1>{}, ic<1 - cur>{});
            const float wv = wb[cur], wpv = wpb[cur];
            float dg[2 * pa.l3 + 1];
            static_range<0, 2 * pa.l3 + 1>([&](auto m) { dg[m] = 0.f; });
            float sw = 0.f;  // dS/dw[e, p, u]
            static_range<pa.pr0, pa.pr1>([&](auto qc) {
                constexpr Pair pr = kTab<L>.pair[qc];
                constexpr int r1 = pa.x_row + pa.l1 + pr.m1, c3 = pr.m3 + pa.l3;
                const float k = pair_coef<L, qc>(Y), kd = pair_coef<L, qc>(Yd);
                const float xm = x[r1], xpm = xp[r1], g = gb[cur][c3];
                const float uy = __builtin_fmaf(wv, xpm, wpv * xm);  // multiplies Y
                const float vy = wv * xm;                            // multiplies Yd
                dg[c3] = __builtin_fmaf(k, uy, __builtin_fmaf(kd, vy, dg[c3]));
                gx[r1] = __builtin_fmaf(g, __builtin_fmaf(wpv, k, wv * kd), gx[r1]);
                sw = __builtin_fmaf(g, __builtin_fmaf(k, xpm, kd * xm), sw);
                const float gu = g * uy, gv = g * vy;
                static_range<pr.t0, pr.t1>([&](auto tc) {
                    constexpr Entry en = kTab<L>.nz[kTab<L>.pair_entries[tc]];
                    constexpr int b = pa.y_row + pa.l2 + en.m2;
                    Z1[b] = __builtin_fmaf(en.fval, gu, Z1[b]);
                    Z2[b] = __builtin_fmaf(en.fval, gv, Z2[b]);
                });
            });
            static_range<0, 2 * pa.l3 + 1>([&](auto m) {
                const uint32_t so = (pa.out_row + m) * rowb;
                float v = dg[m];
                if constexpr (ACC)
                    v += bload<float>(rdg, vo, so);
                bstore<float, kNT>(v, rdg, vo, so);
            });
            {
                float v = sw;
                if constexpr (ACC)
                    v += bload<float>(rdw, vo, pc * rowb);
                bstore<float, kNT>(v, rdw, vo, pc * rowb);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        static_range<0, DIN>([&](auto r) {
            float v = gx[r];
            if constexpr (ACC)
                v += bload<float>(rdv, vo, r * rowb);
            bstore<float, kNT>(v, rdv, vo, r * rowb);
        });
    }
    if (dr) {
        float g0 = 0.f, g1 = 0.f, g2 = 0.f;
        static_range<0, DSH>([&](auto b) {
            Z1[b] = wave_sum_to_lane63(Z1[b]);
            Z2[b] = wave_sum_to_lane63(Z2[b]);
        });
        sh_jet_emit<L>(rx, ry, rz, px, py, pz, [&](auto b, const Jet &y) {
            g0 = __builtin_fmaf(Z1[b], y.b0, __builtin_fmaf(Z2[b], y.d0, g0));
            g1 = __builtin_fmaf(Z1[b], y.b1, __builtin_fmaf(Z2[b], y.d1, g1));
            g2 = __builtin_fmaf(Z1[b], y.b2, __builtin_fmaf(Z2[b], y.d2, g2));
        });
        if (lane == 63) {
            float *ge = dr + 3 * e;
            if constexpr (ACC) {
                g0 += ge[0];
                g1 += ge[1];
                g2 += ge[2];
            }
            ge[0] = g0;
            ge[1] = g1;
            ge[2] = g2;
        }
    }
}

// This file is compiled once per l_max (-DETP_L=0..4, in parallel); the
// C-ABI layer dispatches on l_max to the instantiation of that unit.
#define ETP_EDGE_TP_LAUNCH(F, ...)                                              \
    if (accumulate)                                                             \
        hipLaunchKernelGGL(HIP_KERNEL_NAME(F<L, true>), __VA_ARGS__);           \
    else                                                                        \
        hipLaunchKernelGGL(HIP_KERNEL_NAME(F<L, false>), __VA_ARGS__);

template <int L>
hipError_t edge_tp_fwd_l(int C, int64_t E, const float *vec, const float *V, const float *w, float *out,
                         bool accumulate, hipStream_t stream)
{
    if (E == 0)
        return hipSuccess;
    const int64_t waves = (E + kEdgeTpRun - 1) / kEdgeTpRun * ((C + 63) / 64);
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
    ETP_EDGE_TP_LAUNCH(edge_tp_fwd_kernel, grid, block, 0, stream, E, C, vec, V, w, out)
    return hipGetLastError();
}

template <int L>
hipError_t edge_tp_vjp_l(int C, int64_t E, const float *vec, const float *V, const float *w, const float *G,
                         float *gV, float *gw, float *gr, bool accumulate, hipStream_t stream)
{
    if (E == 0)
        return hipSuccess;
    const dim3 grid(static_cast<unsigned>((E + 3) / 4)), block(256);
    ETP_EDGE_TP_LAUNCH(edge_tp_vjp_kernel, grid, block, 0, stream, E, C, vec, V, w, G, gV, gw, gr)
    return hipGetLastError();
}

template <int L>
hipError_t edge_tp_vjp2_l(int C, int64_t E, const float *vec, const float *V, const float *w, const float *G,
                          const float *ggV, const float *ggw, const float *ggvec, float *dV, float *dw, float *dr,
                          float *dG, bool accumulate, hipStream_t stream)
{
    if (E == 0)
        return hipSuccess;
    const dim3 grid(static_cast<unsigned>((E + 3) / 4)), block(256);
    ETP_EDGE_TP_LAUNCH(edge_tp_vjp2_kernel, grid, block, 0, stream, E, C, vec, V, w, G, ggV, ggw, ggvec, dV, dw,
                       dr, dG)
    return hipGetLastError();
}

#ifndef ETP_L
#error "etp_edge_tp.hip is compiled once per l_max: -DETP_L=<0..4>"
#endif
template hipError_t edge_tp_fwd_l<ETP_L>(int, int64_t, const float *, const float *, const float *, float *, bool,
                                         hipStream_t);
template hipError_t edge_tp_vjp_l<ETP_L>(int, int64_t, const float *, const float *, const float *, const float *,
                                         float *, float *, float *, bool, hipStream_t);
template hipError_t edge_tp_vjp2_l<ETP_L>(int, int64_t, const float *, const float *, const float *,
                                          const float *, const float *, const float *, const float *, float *,
                                          float *, float *, float *, bool, hipStream_t);

}  // namespace etp
