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
