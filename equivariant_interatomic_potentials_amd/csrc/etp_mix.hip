// etp_mix.hip -- the per-irrep channel-mixing linear layer that follows the
// convolution, and its VJP, on the matrix cores.
//
//   y[i, l, m, v] = sum_{p: l3_p = l} sum_u W_l[(q_p C + u), v] out[i, off_p + m, u]
//   gin[i, off_p + m, u] = sum_v W_l[(q_p C + u), v] gy[i, l*l + m, v]
//
// (q_p = rank of path p among the paths of output order l, in path order;
// W = W_0, W_1, ... back to back, W_l of n_l * C rows and C columns; y has
// the node-feature layout [n][(l_max + 1)^2][C], so it can feed the next
// convolution.) The pages name a single dense channel contraction after the
// tensor product, in mixed precision ("Scaling the leading accuracy of deep
// equivariant models to biomolecular simulations of realistic size",
// section "Proposed method"), without fixing its form; one matrix per
// output order, shared by its 2l + 1 components, is the plainest
// equivariant reading.
//
// Per order l the forward is one dense product [n (2l+1)] x [n_l C] times
// [n_l C] x C; the VJP is, per path, [n (2l+1)] x C times C x C (W_{l,q}
// transposed). Mapping (gfx950, wave64):
//   * a workgroup owns 64 rows (node, m) of one order and 64 output
//     channels; 4 waves of 16 rows each hold four 16 x 16 fp32 accumulator
//     tiles; with KW > 1, KW groups of 4 such waves share the tile and take
//     alternate chunks of K, and groups 1.. hand their tiles to group 0
//     through LDS at the end, added in group order (more waves per SIMD and
//     shorter chains on small grids; the result does not depend on timing);
//   * K runs in chunks of 32 channels. Lane (row r = lane % 16, quarter
//     kq = lane / 16) loads the 8 consecutive channels 8 kq .. 8 kq + 7 of
//     the chunk from its A row (two 16-byte loads); the chunk of W (32 x 64)
//     is staged in a double-buffered LDS tile Bt[column][k] (transposed for
//     the forward, whose W rows run along the output channel; as read for
//     the VJP, whose W rows run along k) so that a lane reads its 8 k values
//     of a column as one 16-byte LDS read; the next chunk is loaded into
//     registers while the current one's products run (one barrier per
//     chunk);
//   * fp32 weights: 8 v_mfma_f32_16x16x4f32 per column tile and chunk (step
//     i takes channel 8 kq + i of the chunk); bf16 weights: A is rounded to
//     bf16 (nearest even) in registers and one v_mfma_f32_16x16x32_bf16 per
//     column tile and chunk takes all 32 channels; fp32 accumulation in
//     both, no atomics; rows, columns and channels past the problem are
//     zero-filled or dropped.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "etp_device.hpp"

namespace etp {

#ifndef ETP_MIX_WG_ROWS
#define ETP_MIX_WG_ROWS 32
#endif

constexpr int kMixMaxPaths = 17;  // most paths of one output order (l_max 4, l3 = 3)

struct MixTab {
    int lout, C, n, Dout, Dy;
    int nlmax;                   // most paths of one order
    int nl[5];                   // paths per output order
    int tiles0[6];               // prefix of 64-row tiles over the orders
    int off[5][kMixMaxPaths];    // first output row of each path of order l
    int64_t wofs[6];             // start of W_l (floats)
};

typedef float mix_f4 __attribute__((ext_vector_type(4)));
typedef __bf16 mix_bf8 __attribute__((ext_vector_type(8)));

constexpr int kMixCols = 64;  // output channels per workgroup

__device__ __forceinline__ uint16_t mix_f2bf(float f)
{
    // round to nearest even (finite inputs)
    const uint32_t u = __float_as_uint(f);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// VJP = false: blockIdx = (64-row tile over the orders, column tile); K over
// (path of the order, input channel u). VJP = true: blockIdx = (tile, column
// tile, path q of the order); K over the output channel v.
template <bool BF, int KW, bool VJP>
__global__ void __launch_bounds__(256 * KW) mix2_kernel(const MixTab tb, const float *__restrict__ A,
                                                        const void *__restrict__ Wv, float *__restrict__ out,
                                                        const int accumulate, const int qg)
{
    constexpr int KS = BF ? 40 : 36;  // Bt row stride (elements): 16-byte aligned rows
    // 32-channel sub-chunks per iteration: two for bf16, whose products are
    // four times shorter, so that each barrier covers as many loads in flight
    constexpr int SUB = BF ? 2 : 1;
    using BT = std::conditional_t<BF, uint16_t, float>;
    constexpr int kBtBytes = 2 * KW * SUB * kMixCols * KS * static_cast<int>(sizeof(BT));
    constexpr int kRedBytes = (KW - 1) * 16 * 64 * 16;  // K-group tiles (a float4 per lane and tile)
    __shared__ __attribute__((aligned(16))) unsigned char smem[kBtBytes > kRedBytes ? kBtBytes : kRedBytes];
    auto Bt = reinterpret_cast<BT (*)[KW][SUB][kMixCols][KS]>(smem);
    // VJP: each wave's 16 x 64 result rows pass through LDS so that they
    // leave as whole 256-byte rows (the VJP's output is its largest stream)
    constexpr int kOS = kMixCols + 4;
    __shared__ __attribute__((aligned(16))) float otile[VJP ? 4 * 16 * kOS : 4];
    // the wave index, known to the compiler as uniform over the wave (so are
    // the chunk, path and order indices that follow from it)
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wv & 3, kg = wv >> 2;  // row group of 16 rows, K group
    // blockIdx.x -> (64-row tile over the orders, path (VJP), column tile):
    // workgroups b and b + 8 run on the same XCD, so b = (g nw + w) 8 + x
    // takes row tile 8 g + x and the w-th (path, column tile) pair: the
    // workgroups that read a row tile's A rows run side by side on one XCD
    // and read them through one L2, while consecutive row tiles (and the
    // orders' unequal tiles) still spread over all XCDs. The grid is padded
    // to whole groups of 8 row tiles (and, for the VJP, to the most paths of
    // an order).
    const int ncol = (tb.C + kMixCols - 1) / kMixCols, nw = VJP ? ncol * qg : ncol;
    const int bx = blockIdx.x, xq = bx >> 3, w8 = xq % nw;
    const int tflat = (xq / nw) * 8 + (bx & 7), ctile = w8 % ncol;
    if (tflat >= tb.tiles0[tb.lout + 1])
        return;  // the whole workgroup: padding of the last group
    int l = 0;
    while (l < tb.lout && tflat >= tb.tiles0[l + 1])
        ++l;
    // VJP: this workgroup's paths are qv, qv + qg, ... below the order's
    // count (qg = 1: all of them, one after another; qg = the most paths of
    // an order: one path)
    const int qv = VJP ? w8 / ncol : 0;
    if (VJP && qv >= tb.nl[l])
        return;  // the whole workgroup: this order has fewer paths
    const int npath = VJP ? (tb.nl[l] - qv + qg - 1) / qg : 1;
    const int tile = tflat - tb.tiles0[l];
    const int d = 2 * l + 1, M = tb.n * d, C = tb.C;
    const int c0 = ctile * kMixCols;
    const int kq = lane >> 4, col = lane & 15;

    const int ra = tile * 64 + rg * 16 + col;
    const bool rok = ra < M;
    const int ia = rok ? ra / d : 0, ma = rok ? ra - ia * d : 0;
    // A rows: the convolution output's rows (forward; the path's block is
    // added per chunk) or the cotangent's order-l rows (VJP)
    const float *abase = VJP ? A + (static_cast<int64_t>(ia) * tb.Dy + l * l + ma) * C
                             : A + (static_cast<int64_t>(ia) * tb.Dout + ma) * C;
    const bool vec4 = (C & 3) == 0 && (reinterpret_cast<uintptr_t>(A) & 15u) == 0;

    mix_f4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = mix_f4{0.f, 0.f, 0.f, 0.f};
    // the tile's results (path q's rows for the VJP): lane l holds rows
    // 4 (l / 16) + rr, column 16 t + l % 16 of each tile
    auto store = [&](int q) {
        if constexpr (VJP) {
            float *ot = otile + rg * (16 * kOS);
            wave_sync_lds();  // this wave's previous reads of its rows are done
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    ot[(4 * kq + rr) * kOS + 16 * t + col] = acc[t][rr];
            wave_sync_lds();
            const bool ovec = (C & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e = lane + 64 * k, row = e >> 4, c4 = (e & 15) * 4;
                const int r = tile * 64 + rg * 16 + row;
                if (r >= M)
                    continue;
                const int i = r / d, m = r - i * d;
                float *dst = out + (static_cast<int64_t>(i) * tb.Dout + tb.off[l][q] + m) * C + c0 + c4;
                const float4 v = *reinterpret_cast<const float4 *>(ot + row * kOS + c4);
                if (ovec && c0 + c4 + 4 <= C) {
                    float4 o = v;
                    if (accumulate) {
                        const float4 p0 = *reinterpret_cast<const float4 *>(dst);
                        o = make_float4(p0.x + v.x, p0.y + v.y, p0.z + v.z, p0.w + v.w);
                    }
                    *reinterpret_cast<float4 *>(dst) = o;
                } else {
                    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (c0 + c4 + j < C)
                            dst[j] = accumulate ? dst[j] + vv[j] : vv[j];
                }
            }
            return;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = c0 + 16 * t + col;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = tile * 64 + rg * 16 + 4 * kq + rr;
                if (r < M && c < C) {
                    const int i = r / d, m = r - (r / d) * d;
                    const int64_t row = VJP ? static_cast<int64_t>(i) * tb.Dout + tb.off[l][q] + m
                                            : static_cast<int64_t>(i) * tb.Dy + l * l + m;
                    float *dst = out + row * C + c;
                    *dst = accumulate ? *dst + acc[t][rr] : acc[t][rr];
                }
            }
        }
    };

    // K group kg takes chunks kg, kg + KW, ...; every wave runs the same
    // number of iterations (one barrier each)
    const int ncu = (C + 32 * SUB - 1) / (32 * SUB), nchunk = (VJP ? npath : tb.nl[l]) * ncu,
              nit = (nchunk + KW - 1) / KW;
    float a_nx[SUB][8];
    BT b_nx[SUB][8];
    // W staging, thread t of a K group (t < 256):
    //   forward fp32: W rows k0 + t / 16 and + 16, columns 4 (t % 16) .. + 3
    //   forward bf16: W row k0 + t / 8, columns 8 (t % 8) .. + 7
    //   VJP:          W row c0 + t % 64, entries k0 + 8 ((t / 64) % 4) .. + 7
    const int t8 = threadIdx.x & 255;
    const int sr = VJP ? t8 & 63 : (BF ? t8 >> 3 : t8 >> 4);        // W row (within the chunk or tile)
    const int sc = VJP ? (t8 >> 6) * 8 : (BF ? 8 * (t8 & 7) : 4 * (t8 & 15));  // first W column
    const bool wal = (C & 7) == 0 && (reinterpret_cast<uintptr_t>(Wv) & 15u) == 0;
    auto fetch = [&](int ci) {
        if (ci >= nchunk) {
#pragma unroll
            for (int j = 0; j < SUB; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    a_nx[j][i] = 0.f;
                    b_nx[j][i] = BT(0);
                }
            return;
        }
        const int q = VJP ? qv + (ci / ncu) * qg : ci / ncu, kc = (ci % ncu) * 32 * SUB;
        const float *arow = VJP ? abase : abase + static_cast<int64_t>(tb.off[l][q]) * C;
        const BT *W = static_cast<const BT *>(Wv) + tb.wofs[l] + static_cast<int64_t>(q) * C * C;
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
            const int k0 = kc + 32 * j;
            const int kb = k0 + 8 * kq;
            if (rok && vec4 && kb + 8 <= C) {
                const float4 v0 = *reinterpret_cast<const float4 *>(arow + kb);
                const float4 v1 = *reinterpret_cast<const float4 *>(arow + kb + 4);
                a_nx[j][0] = v0.x; a_nx[j][1] = v0.y; a_nx[j][2] = v0.z; a_nx[j][3] = v0.w;
                a_nx[j][4] = v1.x; a_nx[j][5] = v1.y; a_nx[j][6] = v1.z; a_nx[j][7] = v1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const bool ok = rok && kb + i < C;
                    const float v = arow[ok ? kb + i : 0];  // in bounds either way
                    a_nx[j][i] = ok ? v : 0.f;
                }
            }
            // element (row, col) of the chunk's W block for this thread, zero past
            // the problem; loads stay in bounds (index 0 when out)
            auto wat = [&](int row, int col) -> BT {
                const bool ok = row < C && col < C;
                const BT v = W[ok ? static_cast<int64_t>(row) * C + col : 0];
                return ok ? v : BT(0);
            };
            if constexpr (VJP) {
                const int row = c0 + sr, col = k0 + sc;
                if (wal && row < C && col + 8 <= C) {
                    const BT *src = W + static_cast<int64_t>(row) * C + col;
                    if constexpr (BF) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(src);
                        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            b_nx[j][2 * i] = static_cast<uint16_t>(w4[i] & 0xFFFFu);
                            b_nx[j][2 * i + 1] = static_cast<uint16_t>(w4[i] >> 16);
                        }
                    } else {
                        const float4 v0 = *reinterpret_cast<const float4 *>(src);
                        const float4 v1 = *reinterpret_cast<const float4 *>(src + 4);
                        b_nx[j][0] = v0.x; b_nx[j][1] = v0.y; b_nx[j][2] = v0.z; b_nx[j][3] = v0.w;
                        b_nx[j][4] = v1.x; b_nx[j][5] = v1.y; b_nx[j][6] = v1.z; b_nx[j][7] = v1.w;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        b_nx[j][i] = wat(row, col + i);
                }
            } else if constexpr (BF) {
                const int row = k0 + sr, col = c0 + sc;
                if (wal && row < C && col + 8 <= C) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(W + static_cast<int64_t>(row) * C + col);
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        b_nx[j][2 * i] = static_cast<uint16_t>(w4[i] & 0xFFFFu);
                        b_nx[j][2 * i + 1] = static_cast<uint16_t>(w4[i] >> 16);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        b_nx[j][i] = wat(row, col + i);
                }
            } else {
                const int row = k0 + sr, col = c0 + sc;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int rh = row + 16 * h;
                    if (wal && rh < C && col + 4 <= C) {
                        const float4 v = *reinterpret_cast<const float4 *>(W + static_cast<int64_t>(rh) * C + col);
                        b_nx[j][4 * h] = v.x; b_nx[j][4 * h + 1] = v.y; b_nx[j][4 * h + 2] = v.z; b_nx[j][4 * h + 3] = v.w;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            b_nx[j][4 * h + i] = wat(rh, col + i);
                    }
                }
            }
        }
    };
    // b_nx into the LDS tile Bt[column][k] of this K group
    auto stage = [&](int buf) {
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
            if constexpr (VJP) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    Bt[buf][kg][j][sr][sc + i] = b_nx[j][i];
            } else if constexpr (BF) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    Bt[buf][kg][j][sc + i][sr] = b_nx[j][i];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Bt[buf][kg][j][sc + i][sr] = b_nx[j][i];
                    Bt[buf][kg][j][sc + i][sr + 16] = b_nx[j][4 + i];
                }
            }
        }
    };
    if (nit > 0)
        fetch(kg);
    for (int it = 0; it < nit; ++it) {
        const int buf = it & 1;
        const bool live = it * KW + kg < nchunk;  // uniform over the wave
        stage(buf);
        float a[SUB][8];
#pragma unroll
        for (int j = 0; j < SUB; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                a[j][i] = a_nx[j][i];
        // one barrier per iteration: the tile stores above are seen by every
        // wave, and the buffer written next (buf ^ 1) was last read before it
        __syncthreads();
        if (it + 1 < nit)
            fetch((it + 1) * KW + kg);
        if (!live)
            continue;
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
            if constexpr (BF) {
                mix_bf8 av;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    av[i] = __builtin_bit_cast(__bf16, mix_f2bf(a[j][i]));
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const mix_bf8 bv = *reinterpret_cast<const mix_bf8 *>(&Bt[buf][kg][j][16 * t + col][8 * kq]);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[t], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float4 b0 = *reinterpret_cast<const float4 *>(&Bt[buf][kg][j][16 * t + col][8 * kq]);
                    const float4 b1 = *reinterpret_cast<const float4 *>(&Bt[buf][kg][j][16 * t + col][8 * kq + 4]);
                    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j][i], bb[i], acc[t], 0, 0, 0);
                }
            }
        }
        if constexpr (VJP && KW == 1) {
            if ((it + 1) % ncu == 0) {  // the path's last chunk: store it, start the next
                store(qv + (it / ncu) * qg);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[t] = mix_f4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    if constexpr (KW > 1) {
        // K groups 1.. hand their tiles to group 0 through LDS (reusing the
        // staging space); group 0 adds them in group order
        auto red = reinterpret_cast<mix_f4 (*)[4][4][64]>(smem);
        __syncthreads();
        if (kg > 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                red[kg - 1][rg][t][lane] = acc[t];
        }
        __syncthreads();
        if (kg > 0)
            return;
#pragma unroll
        for (int g = 1; g < KW; ++g) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[t] += red[g - 1][rg][t][lane];
        }
    }

    // (the VJP with one K group stored each path as it finished)
    if constexpr (!VJP || KW > 1)
        store(qv);
}

// Weight gradient of the mixing (the sum over nodes that training needs):
//   gW_l[(q C + u), v] = sum_{i, m} in[i, off_q + m, u] gy[i, l*l + m, v]
// per path q of order l: a product [C] x [n (2l+1)] times [n (2l+1)] x [C]
// whose long K runs over (node, component) rows. blockIdx.x = (path, 64-row
// block of u, 64-column block of v), blockIdx.y = split s of K: the split
// takes the nodes [n s / S, n (s + 1) / S) and writes its partial block to
// part[s] (or, with S = 1, the result to gW); 4 waves of 16 u rows hold
// four 16 x 16 accumulator tiles each (v_mfma_f32_16x16x4f32).
//   * K in chunks of 32 rows: one component m of 32 nodes; chunk row
//     r = 4 st + kq is K step st's row for lane quarter kq;
//   * A (the input's channels u) is read by one wave only: each lane loads
//     its channel of its 8 rows straight from memory (16 lanes, 64
//     contiguous bytes per row); B (the cotangent's 64 channels v, shared by
//     the 4 waves) is loaded with 16-byte loads into a double-buffered LDS
//     tile Bs[row][col][t] laid out so that a lane reads its four column
//     tiles' values as one 16-byte LDS read; the next chunk loads into
//     registers while the current chunk's products run (one barrier per
//     chunk).
constexpr int kMixWgRows = ETP_MIX_WG_ROWS;  // K rows per chunk (a component of that many nodes)
constexpr int kMixWgBS = 68;  // Bs row stride (floats): 16-byte rows, banks shifted per row

struct MixWgTab {
    int P, C, n, Dout, Dy, nub, nvb, nsplit;
    int l3[kMixMaxPaths * 5];      // order of each path
    int off[kMixMaxPaths * 5];     // first output row of each path
    int64_t wofs[kMixMaxPaths * 5];  // start of each path's block in gW
};

__global__ void __launch_bounds__(256) mix_wgrad_kernel(const MixWgTab tb, const float *__restrict__ in,
                                                        const float *__restrict__ gy, float *__restrict__ out,
                                                        const int accumulate)
{
    __shared__ __attribute__((aligned(16))) float Bs[2][kMixWgRows * kMixWgBS];
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kq = lane >> 4, col = lane & 15;
    const int blk = blockIdx.x, s = blockIdx.y;
    const int vb = blk % tb.nvb, ub = (blk / tb.nvb) % tb.nub, p = blk / (tb.nvb * tb.nub);
    const int l = tb.l3[p], d = 2 * l + 1, C = tb.C;
    const int u0 = ub * 64, v0 = vb * 64;
    const int i0 = static_cast<int>(static_cast<int64_t>(tb.n) * s / tb.nsplit);
    const int i1 = static_cast<int>(static_cast<int64_t>(tb.n) * (s + 1) / tb.nsplit);
    const bool vec4 = (C & 3) == 0 && (reinterpret_cast<uintptr_t>(gy) & 15u) == 0;
    const int u = u0 + 16 * wv + col;
    const bool uok = u < C;

    mix_f4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        acc[t] = mix_f4{0.f, 0.f, 0.f, 0.f};

    // A (this wave's 16 u rows; no other wave reads them): the lane loads its
    // channel u of chunk rows 4 st + kq straight from memory. B: thread t
    // stages chunk rows t / 16 + 16 h, channels 4 (t % 16) .. + 3.
    constexpr int NS = kMixWgRows / 4, NH = kMixWgRows / 16;  // K steps, staged rows per thread
    const int sr = threadIdx.x >> 4, sc = 4 * (threadIdx.x & 15);
    float na[NS], nb[NH][4];
    const int nblk = (i1 - i0 + kMixWgRows - 1) / kMixWgRows, nit = nblk * d;
    auto fetch = [&](int it) {
        const int ib = i0 + (it / d) * kMixWgRows, m = it % d;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int i = ib + 4 * st + kq;
            const bool ok = i < i1 && uok;
            const int64_t ic = i < i1 ? i : i0;  // rows past the split load a valid row, then count 0
            const float v = in[(ic * tb.Dout + tb.off[p] + m) * C + (uok ? u : 0)];
            na[st] = ok ? v : 0.f;
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int i = ib + sr + 16 * h;
            const bool iok = i < i1;
            const int64_t ic = iok ? i : i0;
            const float *brow = gy + (ic * tb.Dy + l * l + m) * C;
            if (vec4 && v0 + sc + 4 <= C) {
                const float4 v = *reinterpret_cast<const float4 *>(brow + v0 + sc);
                nb[h][0] = iok ? v.x : 0.f; nb[h][1] = iok ? v.y : 0.f;
                nb[h][2] = iok ? v.z : 0.f; nb[h][3] = iok ? v.w : 0.f;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ok = iok && v0 + sc + j < C;
                    const float v = brow[ok ? v0 + sc + j : 0];  // in bounds either way
                    nb[h][j] = ok ? v : 0.f;
                }
            }
        }
    };
    if (nit > 0)
        fetch(0);
    for (int it = 0; it < nit; ++it) {
        const int buf = it & 1;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int r = sr + 16 * h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int v = sc + j;
                Bs[buf][r * kMixWgBS + (v & 15) * 4 + (v >> 4)] = nb[h][j];
            }
        }
        float av[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st)
            av[st] = na[st];
        // one barrier per chunk: the stores above are seen by every wave,
        // and the buffer written next (buf ^ 1) was last read before it
        __syncthreads();
        if (it + 1 < nit)
            fetch(it + 1);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const float4 bv = *reinterpret_cast<const float4 *>(&Bs[buf][(4 * st + kq) * kMixWgBS + col * 4]);
            acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[st], bv.x, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[st], bv.y, acc[1], 0, 0, 0);
            acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[st], bv.z, acc[2], 0, 0, 0);
            acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[st], bv.w, acc[3], 0, 0, 0);
        }
    }

    // lane l holds u rows 4 (l / 16) + rr of the wave's 16, v column 16 t + l % 16
    float *dst0 = tb.nsplit > 1 ? out + static_cast<int64_t>(s) * tb.wofs[tb.P] : out;
    const bool add = tb.nsplit == 1 && accumulate;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int v = v0 + 16 * t + col;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int uu = u0 + wv * 16 + 4 * kq + rr;
            if (uu < C && v < C) {
                float *o = dst0 + tb.wofs[p] + static_cast<int64_t>(uu) * C + v;
                *o = add ? *o + acc[t][rr] : acc[t][rr];
            }
        }
    }
}

// gW (+)= sum over s < nsplit of part[s] (in order of s), count floats each.
__global__ void __launch_bounds__(256) mix_wgrad_sum_kernel(const int64_t count, const int nsplit,
                                                            const float *__restrict__ part, float *__restrict__ gW,
                                                            const int accumulate)
{
    for (int64_t t = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; t < count;
         t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        float v = 0.f;
        for (int s = 0; s < nsplit; ++s)
            v += part[s * count + t];
        gW[t] = accumulate ? gW[t] + v : v;
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
    tb.nlmax = 1;
    for (int l = 0; l <= L; ++l)
        tb.nlmax = tb.nl[l] > tb.nlmax ? tb.nl[l] : tb.nlmax;
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

// K groups per workgroup: more waves per SIMD and shorter chains when the
// grid alone would leave the SIMDs with one or two waves each (chosen from
// timings of the micro, water and diamond shapes).
static int mix_kgroups(int64_t wgs)
{
    return wgs >= 2048 ? 1 : (wgs >= 640 ? 2 : 4);
}

template <bool VJP>
static hipError_t launch_mix2(int L, int C, int n, const float *A, const void *W, bool bf16, float *out,
                              bool accumulate, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    MixTab tb;
    if (!mix_table_for(L, C, n, &tb))
        return hipErrorInvalidValue;
    const int ncol = (C + kMixCols - 1) / kMixCols;
    // workgroups: one per (row tile, column tile); the VJP also gives each
    // path its own workgroup (qg = most paths of an order) unless that grid
    // is large enough without (qg = 1: a workgroup walks all its order's
    // paths, storing each as it finishes)
    const int64_t tiles = static_cast<int64_t>(tb.tiles0[L + 1]) * ncol;
    int qg = 1, kw = mix_kgroups(tiles);
    if (VJP && kw > 1) {
        qg = tb.nlmax;
        int64_t live = 0;  // workgroups past an order's path count leave at once
        for (int l = 0; l <= L; ++l)
            live += static_cast<int64_t>(ncol) * (tb.tiles0[l + 1] - tb.tiles0[l]) * tb.nl[l];
        kw = mix_kgroups(live);
    }
    const int64_t nwg = static_cast<int64_t>((tb.tiles0[L + 1] + 7) / 8) * 8 * ncol * qg;
    if (nwg > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(nwg));
    const int acc = accumulate ? 1 : 0;
#define ETP_MIX2(BF, KWV)                                                                                            \
    hipLaunchKernelGGL((mix2_kernel<BF, KWV, VJP>), grid, dim3(256 * KWV), 0, stream, tb, A, W, out, acc, qg)
    if (bf16) {
        if (kw == 4)
            ETP_MIX2(true, 4);
        else if (kw == 2)
            ETP_MIX2(true, 2);
        else
            ETP_MIX2(true, 1);
    } else {
        if (kw == 4)
            ETP_MIX2(false, 4);
        else if (kw == 2)
            ETP_MIX2(false, 2);
        else
            ETP_MIX2(false, 1);
    }
#undef ETP_MIX2
    return hipGetLastError();
}

hipError_t launch_mix(int L, int C, int n, const float *in, const void *W, bool bf16, float *y, bool accumulate,
                      hipStream_t stream)
{
    return launch_mix2<false>(L, C, n, in, W, bf16, y, accumulate, stream);
}

hipError_t launch_mix_vjp(int L, int C, int n, const float *gy, const void *W, bool bf16, float *gin,
                          bool accumulate, hipStream_t stream)
{
    return launch_mix2<true>(L, C, n, gy, W, bf16, gin, accumulate, stream);
}

// Splits of the weight gradient's K over the nodes: enough workgroups to
// fill the chip a few times over, each split at least 64 nodes.
static int mix_wgrad_splits(int L, int C, int n)
{
    MixTab tb;
    if (n <= 0 || !mix_table_for(L, C, n, &tb))
        return 1;
    int P = 0;
    for (int l = 0; l <= L; ++l)
        P += tb.nl[l];
    const int64_t tiles = static_cast<int64_t>(P) * ((C + 63) / 64) * ((C + 63) / 64);
    int64_t s = (2048 + tiles - 1) / tiles;
    const int64_t by_nodes = n / 64;  // at least 64 nodes per split
    s = s < by_nodes ? s : by_nodes;
    s = s < 1 ? 1 : (s > 64 ? 64 : s);
    return static_cast<int>(s);
}

size_t mix_wgrad_workspace_bytes(int L, int C, int n)
{
    MixTab tb;
    if (n <= 0 || !mix_table_for(L, C, n, &tb))
        return 0;
    const int S = mix_wgrad_splits(L, C, n);
    return S > 1 ? sizeof(float) * static_cast<size_t>(S) * static_cast<size_t>(tb.wofs[L + 1]) : 0;
}

hipError_t launch_mix_wgrad(int L, int C, int n, const float *in, const float *gy, float *gW, bool accumulate,
                            float *ws, size_t ws_bytes, hipStream_t stream)
{
    MixTab mt;
    if (!mix_table_for(L, C, n, &mt))
        return hipErrorInvalidValue;
    MixWgTab tb{};
    tb.C = C;
    tb.n = n;
    tb.Dout = mt.Dout;
    tb.Dy = mt.Dy;
    tb.nub = (C + 63) / 64;
    tb.nvb = tb.nub;
    int P = 0;
    for (int l = 0; l <= L; ++l)
        for (int q = 0; q < mt.nl[l]; ++q) {
            tb.l3[P] = l;
            tb.off[P] = mt.off[l][q];
            tb.wofs[P] = mt.wofs[l] + static_cast<int64_t>(q) * C * C;
            ++P;
        }
    tb.P = P;
    tb.wofs[P] = mt.wofs[L + 1];
    const int64_t count = mt.wofs[L + 1];
    if (n == 0) {  // an empty sum: zero (or leave the accumulated gradient)
        if (accumulate)
            return hipSuccess;
        const int64_t blocks = (count + 255) / 256;
        hipLaunchKernelGGL(mix_wgrad_sum_kernel, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)),
                           dim3(256), 0, stream, count, 0, ws, gW, 0);
        return hipGetLastError();
    }
    int S = mix_wgrad_splits(L, C, n);
    if (S > 1 && (!ws || ws_bytes < mix_wgrad_workspace_bytes(L, C, n)))
        S = 1;
    tb.nsplit = S;
    const dim3 grid(static_cast<unsigned>(P * tb.nub * tb.nvb), S);
    hipLaunchKernelGGL(mix_wgrad_kernel, grid, dim3(256), 0, stream, tb, in, gy, S > 1 ? ws : gW,
                       accumulate ? 1 : 0);
    if (S > 1) {
        const int64_t blocks = (count + 255) / 256;
        hipLaunchKernelGGL(mix_wgrad_sum_kernel, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)),
                           dim3(256), 0, stream, count, S, ws, gW, accumulate ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace etp
