// etp_mix.hip -- the per-irrep channel-mixing linear layer that follows the
// convolution, on the matrix cores.
//
//   y[i, l, m, v] = sum_{p: l3_p = l} sum_u W_l[(q_p C + u), v] out[i, off_p + m, u]
//
// (q_p = rank of path p among the paths of output order l, in path order;
// W = W_0, W_1, ... back to back, W_l of n_l * C rows and C columns; y has
// the node-feature layout [n][(l_max + 1)^2][C], so it can feed the next
// convolution.) The pages name a single dense channel contraction after the
// tensor product ("Scaling the leading accuracy of deep equivariant models
// to biomolecular simulations of realistic size", section "Proposed
// method") without fixing its form; one matrix per output order, shared by
// its 2l + 1 components, is the plainest equivariant reading.
//
// Per order l it is one dense product [n (2l+1)] x [n_l C] times [n_l C] x C.
// Mapping (gfx950, wave64, v_mfma_f32_16x16x4f32):
//   * a workgroup of 4 waves owns 64 rows (node, m) of one order and 64
//     output channels; each wave owns 16 rows and holds four 16 x 16 fp32
//     accumulator tiles;
//   * K runs over (path of order l, input channel) in chunks of 32 input
//     channels: the chunk of W_l (32 x 64) is staged in a double-buffered
//     LDS tile once per workgroup; each wave reads its A operand straight
//     from the convolution output (lane l: row l % 16, k = l / 16 + 4 s);
//     the next chunk's A and W values are loaded into registers while the
//     current chunk's MFMAs run (one barrier per chunk);
//   * fp32 in, fp32 accumulate, no atomics; rows, output channels and input
//     channels past the problem are zero-filled or dropped.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "etp_tables.hpp"

namespace etp {

constexpr int kMixMaxPaths = 17;  // most paths of one output order (l_max 4, l3 = 3)

struct MixTab {
    int lout, C, n, Dout, Dy;
    int nl[5];                   // paths per output order
    int tiles0[6];               // prefix of 64-row tiles over the orders
    int off[5][kMixMaxPaths];    // first output row of each path of order l
    int64_t wofs[6];             // start of W_l (floats)
};

typedef float mix_f4 __attribute__((ext_vector_type(4)));

constexpr int kMixCols = 64;  // output channels per workgroup

__global__ void __launch_bounds__(256) mix_kernel(const MixTab tb, const float *__restrict__ in,
                                                  const float *__restrict__ W, float *__restrict__ y,
                                                  const int accumulate)
{
    __shared__ float Bs[2][32][kMixCols + 4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int l = 0;
    while (l < tb.lout && static_cast<int>(blockIdx.x) >= tb.tiles0[l + 1])
        ++l;
    const int tile = blockIdx.x - tb.tiles0[l];
    const int d = 2 * l + 1, M = tb.n * d, C = tb.C;
    const int c0 = blockIdx.y * kMixCols;
    const int kq = lane >> 4, col = lane & 15;

    // this lane's A row
    const int ra = tile * 64 + wv * 16 + col;
    const bool rok = ra < M;
    const int ia = rok ? ra / d : 0, ma = rok ? ra - ia * d : 0;
    const float *abase = in + (static_cast<int64_t>(ia) * tb.Dout + ma) * C;

    mix_f4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = mix_f4{0.f, 0.f, 0.f, 0.f};

    // K in chunks of 32 input channels of one path: chunk ci = (q, u0).
    // The next chunk's A and W values are loaded into registers while the
    // current chunk's MFMAs run; W goes through a double-buffered LDS tile.
    const int ncu = (C + 31) / 32, nchunk = tb.nl[l] * ncu;
    constexpr int BPT = 32 * kMixCols / 256;  // W values staged per thread
    float a_nx[8], b_nx[BPT];
    auto fetch = [&](int ci) {
        const int q = ci / ncu, u0 = (ci - q * ncu) * 32;
        const float *arow = abase + static_cast<int64_t>(tb.off[l][q]) * C;
        const float *Wq = W + tb.wofs[l] + static_cast<int64_t>(q) * C * C;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int u = u0 + 4 * s + kq;
            a_nx[s] = (rok && u < C) ? arow[u] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int t = threadIdx.x + 256 * k;
            const int kr = t / kMixCols, cc = t % kMixCols;
            const int u = u0 + kr, c = c0 + cc;
            b_nx[k] = (u < C && c < C) ? Wq[static_cast<int64_t>(u) * C + c] : 0.f;
        }
    };
    fetch(0);
    for (int ci = 0; ci < nchunk; ++ci) {
        const int buf = ci & 1;
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int t = threadIdx.x + 256 * k;
            Bs[buf][t / kMixCols][t % kMixCols] = b_nx[k];
        }
        float a[8];
#pragma unroll
        for (int s = 0; s < 8; ++s)
            a[s] = a_nx[s];
        // one barrier per chunk: the stores above are seen by every wave,
        // and the buffer written next (buf ^ 1) was last read before it
        __syncthreads();
        if (ci + 1 < nchunk)
            fetch(ci + 1);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], Bs[buf][4 * s + kq][16 * t + col], acc[t], 0,
                                                              0, 0);
        }
    }

    // lane l holds rows 4 (l / 16) + rr, column 16 t + l % 16 of each tile
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int c = c0 + 16 * t + col;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = tile * 64 + wv * 16 + 4 * kq + rr;
            if (r < M && c < C) {
                const int i = r / d, m = r - (r / d) * d;
                float *dst = y + (static_cast<int64_t>(i) * tb.Dy + l * l + m) * C + c;
                *dst = accumulate ? *dst + acc[t][rr] : acc[t][rr];
            }
        }
    }
}

// VJP with respect to the input (the mixing is linear: the transposed map):
//   gin[i, off_p + m, u] = sum_v W_l[(q_p C + u), v] gy[i, l*l + m, v]
// per order l and path q one product [n (2l+1)] x C times C x C (W_{l,q}
// transposed). Same tiling as the forward; blockIdx.y = (path q of order l,
// 64-column tile); the W chunk is read along v (contiguous) and transposed
// into the LDS tile.
__global__ void __launch_bounds__(256) mix_vjp_kernel(const MixTab tb, const float *__restrict__ gy,
                                                      const float *__restrict__ W, float *__restrict__ gin,
                                                      const int accumulate)
{
    __shared__ float Bs[2][32][kMixCols + 4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int l = 0;
    while (l < tb.lout && static_cast<int>(blockIdx.x) >= tb.tiles0[l + 1])
        ++l;
    const int C = tb.C, ntc = (C + kMixCols - 1) / kMixCols;
    const int q = blockIdx.y / ntc, c0 = (blockIdx.y - q * ntc) * kMixCols;
    if (q >= tb.nl[l])
        return;  // the whole workgroup: this order has fewer paths
    const int tile = blockIdx.x - tb.tiles0[l];
    const int d = 2 * l + 1, M = tb.n * d;
    const int kq = lane >> 4, col = lane & 15;

    const int ra = tile * 64 + wv * 16 + col;
    const bool rok = ra < M;
    const int ia = rok ? ra / d : 0, ma = rok ? ra - ia * d : 0;
    const float *arow = gy + (static_cast<int64_t>(ia) * tb.Dy + l * l + ma) * C;
    const float *Wq = W + tb.wofs[l] + static_cast<int64_t>(q) * C * C;

    mix_f4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = mix_f4{0.f, 0.f, 0.f, 0.f};

    const int nchunk = (C + 31) / 32;
    constexpr int BPT = 32 * kMixCols / 256;
    float a_nx[8], b_nx[BPT];
    auto fetch = [&](int ci) {
        const int v0 = ci * 32;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
            const int v = v0 + 4 * s8 + kq;
            a_nx[s8] = (rok && v < C) ? arow[v] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int t = threadIdx.x + 256 * k;
            const int kr = t & 31, cc = t >> 5;  // consecutive threads read consecutive v
            const int v = v0 + kr, u = c0 + cc;
            b_nx[k] = (v < C && u < C) ? Wq[static_cast<int64_t>(u) * C + v] : 0.f;
        }
    };
    fetch(0);
    for (int ci = 0; ci < nchunk; ++ci) {
        const int buf = ci & 1;
#pragma unroll
        for (int k = 0; k < BPT; ++k) {
            const int t = threadIdx.x + 256 * k;
            Bs[buf][t & 31][t >> 5] = b_nx[k];
        }
        float a[8];
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8)
            a[s8] = a_nx[s8];
        __syncthreads();
        if (ci + 1 < nchunk)
            fetch(ci + 1);
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s8], Bs[buf][4 * s8 + kq][16 * t + col], acc[t], 0,
                                                              0, 0);
        }
    }

#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int c = c0 + 16 * t + col;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = tile * 64 + wv * 16 + 4 * kq + rr;
            if (r < M && c < C) {
                const int i = r / d, m = r - (r / d) * d;
                float *dst = gin + (static_cast<int64_t>(i) * tb.Dout + tb.off[l][q] + m) * C + c;
                *dst = accumulate ? *dst + acc[t][rr] : acc[t][rr];
            }
        }
    }
}

// Path layout of one l_max for the mixing (from the compile-time table).
template <int L>
static MixTab mix_table(int C, int n)
{
    const Table &T = kTab<L>;
    MixTab tb{};
    tb.lout = L;
    tb.C = C;
    tb.n = n;
    tb.Dout = T.dout_rows;
    tb.Dy = (L + 1) * (L + 1);
    for (int p = 0; p < T.P; ++p) {
        const int l3 = T.path[p].l3;
        tb.off[l3][tb.nl[l3]++] = T.path[p].out_row;
    }
    tb.tiles0[0] = 0;
    tb.wofs[0] = 0;
    for (int l = 0; l <= L; ++l) {
        const int64_t rows = static_cast<int64_t>(n) * (2 * l + 1);
        tb.tiles0[l + 1] = tb.tiles0[l] + static_cast<int>((rows + 63) / 64);
        tb.wofs[l + 1] = tb.wofs[l] + static_cast<int64_t>(tb.nl[l]) * C * C;
    }
    return tb;
}

static bool mix_table_for(int L, int C, int n, MixTab *tb)
{
    switch (L) {
    case 0: *tb = mix_table<0>(C, n); return true;
    case 1: *tb = mix_table<1>(C, n); return true;
    case 2: *tb = mix_table<2>(C, n); return true;
    case 3: *tb = mix_table<3>(C, n); return true;
    case 4: *tb = mix_table<4>(C, n); return true;
    default: return false;
    }
}

hipError_t launch_mix(int L, int C, int n, const float *in, const float *W, float *y, bool accumulate,
                      hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    MixTab tb;
    if (!mix_table_for(L, C, n, &tb))
        return hipErrorInvalidValue;
    const dim3 grid(tb.tiles0[L + 1], (C + kMixCols - 1) / kMixCols);
    hipLaunchKernelGGL(mix_kernel, grid, dim3(256), 0, stream, tb, in, W, y, accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_mix_vjp(int L, int C, int n, const float *gy, const float *W, float *gin, bool accumulate,
                          hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    MixTab tb;
    if (!mix_table_for(L, C, n, &tb))
        return hipErrorInvalidValue;
    int maxnl = 0;
    for (int l = 0; l <= L; ++l)
        maxnl = tb.nl[l] > maxnl ? tb.nl[l] : maxnl;
    const dim3 grid(tb.tiles0[L + 1], maxnl * ((C + kMixCols - 1) / kMixCols));
    hipLaunchKernelGGL(mix_vjp_kernel, grid, dim3(256), 0, stream, tb, gy, W, gin, accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace etp
