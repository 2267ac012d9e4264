// etp_conv_common.hpp -- pieces shared by the convolution kernels: launch
// descriptors, per-(l_max, channels-per-lane) tuning, the per-edge
// coefficient table T = sum_m2 C Y_m2 written to LDS, and the
// deterministic cross-wave reduction.
#pragma once
#include <hip/hip_runtime.h>

#include "etp_device.hpp"
#include "etp_groups.hpp"

namespace etp {

// Arguments of every convolution launch (fields a pass does not use are
// null). out is the destination-pass output (out or dG); ox / ow / ovec are
// the source-pass outputs (grad_x / grad_w / grad_vec or d_x / d_w / d_vec).
struct ConvArgs {
    int C;
    int n_dst, n_src;
    const int *row_ptr, *src, *src_ptr, *perm, *perm_dst;
    const float *vec;
    const void *x;
    const float *w, *G, *ggx, *ggw, *ggvec;
    float *out, *ox, *ow, *ovec;
    const float *h, *wr;  // radial features [E][nbasis] and last-layer matrix [nbasis][P][C]
    const float *ggh;     // radial VJP-of-VJP: cotangent on grad_h [E][nbasis]
    float *oh;            // radial VJP: grad_h [E][nbasis] (VJP-of-VJP: d_h)
    float *owr;           // radial weight gradient: per-source-node partials [n_src][8][P][C]
    int nbasis;
    uint32_t flags;
    hipStream_t stream;
};

enum { DST_FWD = 0, DST_DG = 1, DST_FWD_RADIAL = 2, DST_DG_RADIAL = 3 };
constexpr int kRadialMax = 8;  // radial basis functions per edge (padded to this in LDS)
// gr / dr partial slices (3 floats per edge each) that the destination-side
// backward's workspace holds after the per-edge part rows: path groups
// 1 .. kBwdGrSlices may then run side by side with group 0
constexpr int kBwdGrSlices = 2;
enum { SRC_VJP = 0, SRC_VJP2 = 1, SRC_VJP_RADIAL = 2, SRC_VJP2_RADIAL = 3, SRC_VJP_RADIAL_WG = 4, SRC_VJP2_RADIAL_WG = 5 };

// Each kernel source is compiled once per (l_max, x dtype, mode) with
// -DETP_L, -DETP_XT (0 = f32, 1 = bf16) and -DETP_MODE, so the translation
// units build in parallel; each defines one of these entry points.
#define ETP_CAT2(a, b) a##b
#define ETP_CAT(a, b) ETP_CAT2(a, b)
#define ETP_RUN_NAME2(kind, L, XT, MODE) run_##kind##_L##L##_X##XT##_M##MODE
#define ETP_RUN_NAME(kind, L, XT, MODE) ETP_RUN_NAME2(kind, L, XT, MODE)
#define ETP_DECLARE_RUN(kind, L, XT, MODE) hipError_t ETP_RUN_NAME(kind, L, XT, MODE)(const ConvArgs &a);
#define ETP_DECLARE_RUN_L(kind, L) \
    ETP_DECLARE_RUN(kind, L, 0, 0) ETP_DECLARE_RUN(kind, L, 0, 1) ETP_DECLARE_RUN(kind, L, 1, 0) ETP_DECLARE_RUN(kind, L, 1, 1)
#define ETP_DECLARE_RUN_RADIAL(L) \
    ETP_DECLARE_RUN(dst, L, 0, 2) ETP_DECLARE_RUN(dst, L, 1, 2) ETP_DECLARE_RUN(dst, L, 0, 3) ETP_DECLARE_RUN(dst, L, 1, 3)
ETP_DECLARE_RUN_RADIAL(0) ETP_DECLARE_RUN_RADIAL(1) ETP_DECLARE_RUN_RADIAL(2) ETP_DECLARE_RUN_RADIAL(3)
ETP_DECLARE_RUN_RADIAL(4)
#define ETP_DECLARE_RUN_SRC_RADIAL(L)                                                                           \
    ETP_DECLARE_RUN(src, L, 0, 2) ETP_DECLARE_RUN(src, L, 1, 2) ETP_DECLARE_RUN(src, L, 0, 3) ETP_DECLARE_RUN(src, L, 1, 3) \
    ETP_DECLARE_RUN(src, L, 0, 4) ETP_DECLARE_RUN(src, L, 1, 4) ETP_DECLARE_RUN(src, L, 0, 5) ETP_DECLARE_RUN(src, L, 1, 5)
ETP_DECLARE_RUN_SRC_RADIAL(0) ETP_DECLARE_RUN_SRC_RADIAL(1) ETP_DECLARE_RUN_SRC_RADIAL(2)
ETP_DECLARE_RUN_SRC_RADIAL(3) ETP_DECLARE_RUN_SRC_RADIAL(4)
ETP_DECLARE_RUN_L(dst, 0) ETP_DECLARE_RUN_L(dst, 1) ETP_DECLARE_RUN_L(dst, 2) ETP_DECLARE_RUN_L(dst, 3) ETP_DECLARE_RUN_L(dst, 4)
ETP_DECLARE_RUN_L(src, 0) ETP_DECLARE_RUN_L(src, 1) ETP_DECLARE_RUN_L(src, 2) ETP_DECLARE_RUN_L(src, 3) ETP_DECLARE_RUN_L(src, 4)

template <int I>
__device__ __forceinline__ float pick4(const float4 &v)
{
    if constexpr (I == 0)
        return v.x;
    else if constexpr (I == 1)
        return v.y;
    else if constexpr (I == 2)
        return v.z;
    else
        return v.w;
}

// T[q] = sum over the pair's entries of C * Y[l2, m2], for the pairs
// [PR0, PR0 + NPR), stored as float4 chunks (zero padded to STRIDE). Each
// chunk is stored as soon as its four values exist, so only a handful of T
// values are live at a time.
template <int L, int PR0, int NPR, int STRIDE>
__device__ __forceinline__ void write_T(const float *Y, float *dst)
{
    float t[4];
    static_range<0, STRIDE>([&](auto ql) {
        if constexpr (ql < NPR) {
            constexpr Pair pr = kTab<L>.pair[PR0 + ql];
            constexpr Path pa = kTab<L>.path[pr.path];
            static_range<pr.t0, pr.t1>([&](auto ti) {
                constexpr Entry en = kTab<L>.nz[kTab<L>.pair_entries[ti]];
                constexpr int yb = pa.y_row + en.m2 + pa.l2;
                if constexpr (ti == pr.t0)
                    t[ql % 4] = en.fval * Y[yb];
                else
                    t[ql % 4] = fmaf(en.fval, Y[yb], t[ql % 4]);
            });
        } else {
            t[ql % 4] = 0.f;
        }
        if constexpr (ql % 4 == 3)
            *reinterpret_cast<float4 *>(dst + ql - 3) = make_float4(t[0], t[1], t[2], t[3]);
    });
}

constexpr int ilog2(int v)
{
    int r = 0;
    while ((1 << r) < v)
        ++r;
    return r;
}

// Sum the S waves' register accumulators into wave 0 through LDS in a fixed
// tree order ((w0 + w2) + (w1 + w3) for S = 4), in row chunks that fit
// LDS_FLOATS.
template <int S, int NROW, typename V, int LDS_FLOATS>
__device__ __forceinline__ void reduce_waves(V (&acc)[NROW], float *lds, int lane, int wv)
{
    constexpr int CPL = sizeof(V) / 4;
    if constexpr (S > 1) {
        static_range<0, ilog2(S)>([&](auto lv) {
            constexpr int h = S >> (lv + 1);
            constexpr int PER_ROW = 64 * CPL;
            constexpr int CAP = LDS_FLOATS / (h * PER_ROW);
            static_assert(CAP >= 1, "LDS too small for the cross-wave reduction");
            constexpr int CH = CAP < NROW ? CAP : NROW;
            constexpr int NCH = (NROW + CH - 1) / CH;
            static_range<0, NCH>([&](auto ch) {
                constexpr int r0 = ch * CH;
                constexpr int r1 = (r0 + CH) < NROW ? (r0 + CH) : NROW;
                __syncthreads();
                if (wv >= h && wv < 2 * h) {
                    float *dst = lds + (wv - h) * (CH * PER_ROW) + lane * CPL;
                    static_range<r0, r1>([&](auto r) { store_v<V>(dst + (r - r0) * PER_ROW, acc[r]); });
                }
                __syncthreads();
                if (wv < h) {
                    const float *sp = lds + wv * (CH * PER_ROW) + lane * CPL;
                    static_range<r0, r1>([&](auto r) { acc[r] += load_cached<V>(sp + (r - r0) * PER_ROW); });
                }
            });
        });
    }
}

}  // namespace etp
