// etp_node_product.hip -- the node-local correlation product: weighted
// products of a node's irreps with themselves, applied step by step, each
// result truncated to orders <= l_max (the node-local product ladder of "How
// does FlashCart make equivariant interatomic potentials faster and more
// accurate?", section "Generated kernels beat SH baselines at high order").
// Channel by channel:
//   B_1 = A
//   B_{k+1}[l3, m3, u] = sum_{p = (l1, l2, l3)} W[k-1][p][u]
//                        sum_{(m1, m2, m3)} C_p[m1, m2, m3] B_k[l1, m1, u] A[l2, m2, u]
//   out = B_1 + ... + B_nu
// over the convolution's path list and real CG table (l1, l2, l3 <= l_max).
//
// Mapping (gfx950, wave64): one lane per (node, channel); a wave holds 64
// channels of one node. A, the current B, the next B and the running sum stay
// in registers for the whole ladder; the CG table is compiled in as
// immediates, grouped by (path, m1, m2) so that each product B[l1, m1] A[l2,
// m2] is formed once and shared by the entries of that group (one FMA each).
// Memory traffic is A in and out once plus the weights (L2-resident), so the
// kernel is bound by the VALU.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "etp_device.hpp"
#include "etp_tables.hpp"

namespace etp {

size_t block_sum_tmp_floats(int total);
hipError_t launch_block_sum(int64_t n, int64_t stride, int total, const float *part, float *tmp, float *out,
                            bool accumulate, hipStream_t stream);

static const Table &table_for_l(int L)
{
    switch (L) {
    case 0: return kTab<0>;
    case 1: return kTab<1>;
    case 2: return kTab<2>;
    case 3: return kTab<3>;
    default: return kTab<4>;
    }
}

// Registers: A, B_k, B_{k+1} and the running sum (4 (l_max+1)^2 values) plus
// a ring of kNpPrefetch weights, slot = path % kNpPrefetch. While path p
// computes, its slot is refilled for its next user (path p + kNpPrefetch, or
// the same slot's first path of the next step),
// and a scheduling barrier after every path keeps the compiler from hoisting
// every load and product of a step at once (which spills at l_max 4).
constexpr int kNpPrefetch = 4;

template <int L>
constexpr int np_waves_per_eu()
{
    return L <= 2 ? 4 : (L == 3 ? 4 : 3);
}

template <int L>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(np_waves_per_eu<L>())))
node_product_kernel(const int n, const int C, const int nu, const float *__restrict__ A, const float *__restrict__ W,
                    float *__restrict__ out, const int accumulate)
{
    constexpr int D = (L + 1) * (L + 1), P = kTab<L>.P, PF = kNpPrefetch;
    const int lane = threadIdx.x & 63;
    const int cw = (C + 63) >> 6;  // waves per node
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
    if (wid >= static_cast<int64_t>(n) * cw)
        return;
    const int i = static_cast<int>(wid / cw);
    const int u = static_cast<int>(wid - static_cast<int64_t>(i) * cw) * 64 + lane;
    const bool ok = u < C;
    const int uc = ok ? u : 0;
    const float *Ai = A + static_cast<int64_t>(i) * D * C + uc;
    // weights through a buffer descriptor: a lane offset plus a wave-uniform
    // row offset, and the range check returns 0 past the last step (and for
    // lanes beyond C)
    const rsrc_t rw = make_rsrc(W, static_cast<uint32_t>((nu - 1) * P * C * 4));
    const uint32_t wv = ok ? static_cast<uint32_t>(u) * 4u : kOOB;
    auto wload = [&](int k, int q) { return bload<float>(rw, wv, static_cast<uint32_t>((k * P + q) * C * 4)); };

    float a[D], b[D], o[D];
    static_range<0, D>([&](auto r) {
        a[r] = ok ? Ai[static_cast<int64_t>(r) * C] : 0.f;
        b[r] = a[r];
        o[r] = a[r];
    });
    float wr[PF];
    static_range<0, PF>([&](auto q) { wr[q] = q < P ? wload(0, q) : 0.f; });
    for (int k = 0; k + 1 < nu; ++k) {
        float nb[D];
        static_range<0, D>([&](auto r) { nb[r] = 0.f; });
        static_range<0, P>([&](auto pc) {
            constexpr int p = pc;
            constexpr Path pa = kTab<L>.path[p];
            const float w = wr[p % PF];
            // refill the freed slot with its next user: path p + PF of this
            // step, else path p % PF of the next step (slot = path % PF)
            if constexpr (p + PF < P)
                wr[p % PF] = wload(k, p + PF);
            else
                wr[p % PF] = wload(k + 1, p % PF);
            float acc[2 * pa.l3 + 1];
            static_range<0, 2 * pa.l3 + 1>([&](auto m) { acc[m] = 0.f; });
            static_range<kTab<L>.path_ab0[p], kTab<L>.path_ab0[p + 1]>([&](auto gc) {
                constexpr ABGroup g = kTab<L>.ab[gc];
                const float t = b[pa.l1 * pa.l1 + pa.l1 + g.m1] * a[pa.l2 * pa.l2 + pa.l2 + g.m2];
                static_range<g.t0, g.t1>([&](auto ec) {
                    constexpr Entry e = kTab<L>.nz[kTab<L>.ab_entries[ec]];
                    acc[e.m3 + pa.l3] = __builtin_fmaf(e.fval, t, acc[e.m3 + pa.l3]);
                });
            });
            static_range<0, 2 * pa.l3 + 1>(
                [&](auto m) { nb[pa.l3 * pa.l3 + m] = __builtin_fmaf(w, acc[m], nb[pa.l3 * pa.l3 + m]); });
            __builtin_amdgcn_sched_barrier(0);
        });
        static_range<0, D>([&](auto r) {
            b[r] = nb[r];
            o[r] += nb[r];
        });
    }
    if (ok) {
        float *oi = out + static_cast<int64_t>(i) * D * C + u;
        static_range<0, D>([&](auto r) {
            float *d = oi + static_cast<int64_t>(r) * C;
            *d = accumulate ? *d + o[r] : o[r];
        });
    }
}

// ---------------------------------------------------------------- VJP (A)
// gA = d<G, out>/dA by reverse mode over the ladder (see the header of the
// oracle's version for the recursion). Each reverse step k needs B_{k+1},
// which is recomputed from A in registers (k forward steps) rather than kept
// for every step: (nu - 1)(nu - 2) / 2 extra forward steps, no memory.

// One forward step nb = sum_p W[k][p] CG_p(b, a), with its own weight ring.
template <int L, typename WL>
__device__ __forceinline__ void np_step(const float *a, const float *b, float *nb, int k, WL &&wload)
{
    constexpr int D = (L + 1) * (L + 1), P = kTab<L>.P, PF = kNpPrefetch;
    float wr[PF];
    static_range<0, PF>([&](auto q) { wr[q] = q < P ? wload(k, q) : 0.f; });
    static_range<0, D>([&](auto r) { nb[r] = 0.f; });
    static_range<0, P>([&](auto pc) {
        constexpr int p = pc;
        constexpr Path pa = kTab<L>.path[p];
        const float w = wr[p % PF];
        if constexpr (p + PF < P)
            wr[p % PF] = wload(k, p + PF);
        float acc[2 * pa.l3 + 1];
        static_range<0, 2 * pa.l3 + 1>([&](auto m) { acc[m] = 0.f; });
        static_range<kTab<L>.path_ab0[p], kTab<L>.path_ab0[p + 1]>([&](auto gc) {
            constexpr ABGroup g = kTab<L>.ab[gc];
            const float t = b[pa.l1 * pa.l1 + pa.l1 + g.m1] * a[pa.l2 * pa.l2 + pa.l2 + g.m2];
            static_range<g.t0, g.t1>([&](auto ec) {
                constexpr Entry e = kTab<L>.nz[kTab<L>.ab_entries[ec]];
                acc[e.m3 + pa.l3] = __builtin_fmaf(e.fval, t, acc[e.m3 + pa.l3]);
            });
        });
        static_range<0, 2 * pa.l3 + 1>(
            [&](auto m) { nb[pa.l3 * pa.l3 + m] = __builtin_fmaf(w, acc[m], nb[pa.l3 * pa.l3 + m]); });
        __builtin_amdgcn_sched_barrier(0);
    });
}

template <int L, bool WG>
constexpr int np_vjp_waves_per_eu()
{
    // (the weight-gradient form holds one more product per group: one step
    // lower in occupancy at l_max >= 3, where it would spill otherwise)
    return L <= 2 ? 4 : (L == 3 ? (WG ? 2 : 3) : (WG ? 1 : 2));
}

// WG: also the weight gradient's per-node partials, gwp[i][k][p][u] =
// sum_{(m1, m2, m3) in p} C Bbar_{k+2}[l3, m3] B_{k+1}[l1, m1] A[l2, m2] for
// forward step k (W[k]), to be summed over the nodes in order afterwards;
// gA is then optional (NULL: not stored).
template <int L, bool ACC, bool WG>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(np_vjp_waves_per_eu<L, WG>())))
node_product_vjp_kernel(const int n, const int C, const int nu, const float *__restrict__ A,
                        const float *__restrict__ W, const float *__restrict__ G, float *__restrict__ gA,
                        float *__restrict__ gwp)
{
    constexpr int D = (L + 1) * (L + 1), P = kTab<L>.P, PF = kNpPrefetch;
    const int lane = threadIdx.x & 63;
    const int cw = (C + 63) >> 6;
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
    if (wid >= static_cast<int64_t>(n) * cw)
        return;
    const int i = static_cast<int>(wid / cw);
    const int u = static_cast<int>(wid - static_cast<int64_t>(i) * cw) * 64 + lane;
    const bool ok = u < C;
    const uint32_t vo = ok ? static_cast<uint32_t>(u) * 4u : kOOB, rowb = static_cast<uint32_t>(C) * 4u;
    const rsrc_t ra = make_rsrc(A + static_cast<int64_t>(i) * D * C, D * rowb);
    const rsrc_t rg = make_rsrc(G + static_cast<int64_t>(i) * D * C, D * rowb);
    const rsrc_t rw = make_rsrc(W, static_cast<uint32_t>((nu - 1) * P * C * 4));
    auto wload = [&](int k, int q) { return bload<float>(rw, vo, static_cast<uint32_t>((k * P + q) * C * 4)); };
    // this node's block of weight-gradient partials ([nu-1][P][C])
    const rsrc_t rgw = make_rsrc(WG ? gwp + static_cast<int64_t>(i) * (nu - 1) * P * C : nullptr,
                                 WG ? static_cast<uint32_t>((nu - 1) * P * C * 4) : 0u);

    float a[D], ga[D], bb[D];
    static_range<0, D>([&](auto r) {
        a[r] = bload<float>(ra, vo, r * rowb);
        bb[r] = bload<float>(rg, vo, r * rowb);  // dL/dB_nu = G
        ga[r] = 0.f;
    });
    for (int k = nu - 2; k >= 0; --k) {
        // B after k forward steps
        float b[D];
        static_range<0, D>([&](auto r) { b[r] = a[r]; });
        for (int j = 0; j < k; ++j) {
            float nb[D];
            np_step<L>(a, b, nb, j, wload);
            static_range<0, D>([&](auto r) { b[r] = nb[r]; });
        }
        // reverse of forward step k: dL/dB (before it) = G + J_b^T bb, gA += J_a^T bb
        float nbb[D];
        static_range<0, D>([&](auto r) { nbb[r] = bload<float>(rg, vo, r * rowb); });
        float wr[PF];
        static_range<0, PF>([&](auto q) { wr[q] = q < P ? wload(k, q) : 0.f; });
        static_range<0, P>([&](auto pc) {
            constexpr int p = pc;
            constexpr Path pa = kTab<L>.path[p];
            const float w = wr[p % PF];
            if constexpr (p + PF < P)
                wr[p % PF] = wload(k, p + PF);
            if constexpr (!WG) {
                float wb[2 * pa.l3 + 1];
                static_range<0, 2 * pa.l3 + 1>([&](auto m) { wb[m] = w * bb[pa.l3 * pa.l3 + m]; });
                static_range<kTab<L>.path_ab0[p], kTab<L>.path_ab0[p + 1]>([&](auto gc) {
                    constexpr ABGroup g = kTab<L>.ab[gc];
                    constexpr int r1 = pa.l1 * pa.l1 + pa.l1 + g.m1, r2 = pa.l2 * pa.l2 + pa.l2 + g.m2;
                    float c = 0.f;
                    static_range<g.t0, g.t1>([&](auto ec) {
                        constexpr Entry e = kTab<L>.nz[kTab<L>.ab_entries[ec]];
                        c = __builtin_fmaf(e.fval, wb[e.m3 + pa.l3], c);
                    });
                    nbb[r1] = __builtin_fmaf(c, a[r2], nbb[r1]);
                    ga[r2] = __builtin_fmaf(c, b[r1], ga[r2]);
                });
            } else {
                // the same with the weight factored out: cq = sum C Bbar (per
                // (m1, m2) group), c = w cq, and the weight's cotangent
                // sum cq B[l1, m1] A[l2, m2] of this node
                float gw = 0.f;
                static_range<kTab<L>.path_ab0[p], kTab<L>.path_ab0[p + 1]>([&](auto gc) {
                    constexpr ABGroup g = kTab<L>.ab[gc];
                    constexpr int r1 = pa.l1 * pa.l1 + pa.l1 + g.m1, r2 = pa.l2 * pa.l2 + pa.l2 + g.m2;
                    float cq = 0.f;
                    static_range<g.t0, g.t1>([&](auto ec) {
                        constexpr Entry e = kTab<L>.nz[kTab<L>.ab_entries[ec]];
                        cq = __builtin_fmaf(e.fval, bb[pa.l3 * pa.l3 + e.m3 + pa.l3], cq);
                    });
                    const float c = w * cq;
                    nbb[r1] = __builtin_fmaf(c, a[r2], nbb[r1]);
                    ga[r2] = __builtin_fmaf(c, b[r1], ga[r2]);
                    gw = __builtin_fmaf(cq, b[r1] * a[r2], gw);
                });
                bstore<float>(gw, rgw, vo, static_cast<uint32_t>((k * P + p) * C * 4));
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        static_range<0, D>([&](auto r) { bb[r] = nbb[r]; });
    }
    if (WG && !gA)
        return;
    const rsrc_t ro = make_rsrc(gA + static_cast<int64_t>(i) * D * C, D * rowb);
    static_range<0, D>([&](auto r) {
        float v = ga[r] + bb[r];  // B_1 = A
        if constexpr (ACC)
            v += bload<float>(ro, vo, r * rowb);
        bstore<float>(v, ro, vo, r * rowb);
    });
}

hipError_t launch_node_product_vjp(int L, int C, int n, int nu, const float *A, const float *W, const float *G,
                                   float *gA, bool accumulate, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const int64_t waves = static_cast<int64_t>(n) * ((C + 63) / 64);
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
#define ETP_NPV_CASE(LL)                                                                                      \
    case LL:                                                                                                  \
        if (accumulate)                                                                                       \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(node_product_vjp_kernel<LL, true, false>), grid, block, 0,     \
                               stream, n, C, nu, A, W, G, gA, nullptr);                                       \
        else                                                                                                  \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(node_product_vjp_kernel<LL, false, false>), grid, block, 0,    \
                               stream, n, C, nu, A, W, G, gA, nullptr);                                       \
        break;
    switch (L) {
        ETP_NPV_CASE(0) ETP_NPV_CASE(1) ETP_NPV_CASE(2) ETP_NPV_CASE(3) ETP_NPV_CASE(4)
    default: return hipErrorInvalidValue;
    }
#undef ETP_NPV_CASE
    return hipGetLastError();
}

// Workspace of the weight gradient: per-node partial blocks of (nu-1) P C
// floats, then the ordered sum's runs.
size_t node_product_wgrad_workspace_bytes(int L, int C, int n, int nu)
{
    if (L < 0 || L > 4 || nu < 2 || n < 0)
        return 0;
    const int P = table_for_l(L).P;
    const int64_t blk = static_cast<int64_t>(nu - 1) * P * C;
    return sizeof(float) * (static_cast<size_t>(n) * blk + block_sum_tmp_floats(static_cast<int>(blk)));
}

hipError_t launch_node_product_wgrad(int L, int C, int n, int nu, const float *A, const float *W, const float *G,
                                     float *gA, float *gW, bool accumulate, float *ws, hipStream_t stream)
{
    const int P = table_for_l(L).P;
    const int64_t blk = static_cast<int64_t>(nu - 1) * P * C;
    if (blk <= 0)
        return hipSuccess;
    if (n > 0) {
        const int64_t waves = static_cast<int64_t>(n) * ((C + 63) / 64);
        const dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
#define ETP_NPW_CASE(LL)                                                                                      \
    case LL:                                                                                                  \
        if (accumulate)                                                                                       \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(node_product_vjp_kernel<LL, true, true>), grid, block, 0,      \
                               stream, n, C, nu, A, W, G, gA, ws);                                            \
        else                                                                                                  \
            hipLaunchKernelGGL(HIP_KERNEL_NAME(node_product_vjp_kernel<LL, false, true>), grid, block, 0,     \
                               stream, n, C, nu, A, W, G, gA, ws);                                            \
        break;
        switch (L) {
            ETP_NPW_CASE(0) ETP_NPW_CASE(1) ETP_NPW_CASE(2) ETP_NPW_CASE(3) ETP_NPW_CASE(4)
        default: return hipErrorInvalidValue;
        }
#undef ETP_NPW_CASE
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // the partials summed over the nodes in index order (with no nodes: zero,
    // or left as they are when accumulating)
    return launch_block_sum(n, blk, static_cast<int>(blk), ws, ws + static_cast<size_t>(n) * blk, gW, accumulate,
                            stream);
}

hipError_t launch_node_product(int L, int C, int n, int nu, const float *A, const float *W, float *out,
                               bool accumulate, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const int64_t waves = static_cast<int64_t>(n) * ((C + 63) / 64);
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
    const int acc = accumulate ? 1 : 0;
    switch (L) {
    case 0: hipLaunchKernelGGL(node_product_kernel<0>, grid, block, 0, stream, n, C, nu, A, W, out, acc); break;
    case 1: hipLaunchKernelGGL(node_product_kernel<1>, grid, block, 0, stream, n, C, nu, A, W, out, acc); break;
    case 2: hipLaunchKernelGGL(node_product_kernel<2>, grid, block, 0, stream, n, C, nu, A, W, out, acc); break;
    case 3: hipLaunchKernelGGL(node_product_kernel<3>, grid, block, 0, stream, n, C, nu, A, W, out, acc); break;
    case 4: hipLaunchKernelGGL(node_product_kernel<4>, grid, block, 0, stream, n, C, nu, A, W, out, acc); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace etp
