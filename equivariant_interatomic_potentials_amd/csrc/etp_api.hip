// etp_api.hip -- the C ABI declared in include/etp.h: plan creation and
// table readback, host-side argument validation, and dispatch to the
// per-l_max kernel launchers.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>

#include "../../include/etp.h"
#include "etp_conv_common.hpp"

namespace etp {

hipError_t launch_sh(int L, int64_t n, const float *vec, float *Y, float *dY, hipStream_t stream);
hipError_t launch_mix(int L, int C, int n, const float *in, const void *W, bool bf16, float *y, bool accumulate,
                      hipStream_t stream);
hipError_t launch_mix_vjp(int L, int C, int n, const float *gy, const void *W, bool bf16, float *gin,
                          bool accumulate, hipStream_t stream);
size_t mix_wgrad_workspace_bytes(int L, int C, int n);
hipError_t launch_mix_wgrad(int L, int C, int n, const float *in, const float *gy, float *gW, bool accumulate,
                            float *ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_node_product(int L, int C, int n, int nu, const float *A, const float *W, float *out,
                               bool accumulate, hipStream_t stream);
// the edge-local product, one translation unit per l_max
template <int L>
hipError_t edge_tp_fwd_l(int C, int64_t E, const float *vec, const float *V, const float *w, float *out,
                         bool accumulate, hipStream_t stream);
template <int L>
hipError_t edge_tp_vjp_l(int C, int64_t E, const float *vec, const float *V, const float *w, const float *G,
                         float *gV, float *gw, float *gr, bool accumulate, hipStream_t stream);
template <int L>
hipError_t edge_tp_vjp2_l(int C, int64_t E, const float *vec, const float *V, const float *w, const float *G,
                          const float *ggV, const float *ggw, const float *ggvec, float *dV, float *dw, float *dr,
                          float *dG, bool accumulate, hipStream_t stream);

#define ETP_BY_L(F, ...)                              \
    switch (L) {                                      \
    case 0: return F<0>(__VA_ARGS__);                 \
    case 1: return F<1>(__VA_ARGS__);                 \
    case 2: return F<2>(__VA_ARGS__);                 \
    case 3: return F<3>(__VA_ARGS__);                 \
    case 4: return F<4>(__VA_ARGS__);                 \
    default: return hipErrorInvalidValue;             \
    }

hipError_t launch_edge_tp_fwd(int L, int C, int64_t E, const float *vec, const float *V, const float *w, float *out,
                              bool accumulate, hipStream_t stream)
{
    ETP_BY_L(edge_tp_fwd_l, C, E, vec, V, w, out, accumulate, stream)
}

hipError_t launch_edge_tp_vjp(int L, int C, int64_t E, const float *vec, const float *V, const float *w,
                              const float *G, float *gV, float *gw, float *gr, bool accumulate, hipStream_t stream)
{
    ETP_BY_L(edge_tp_vjp_l, C, E, vec, V, w, G, gV, gw, gr, accumulate, stream)
}
size_t node_product_wgrad_workspace_bytes(int L, int C, int n, int nu);
hipError_t launch_node_product_wgrad(int L, int C, int n, int nu, const float *A, const float *W, const float *G,
                                     float *gA, float *gW, bool accumulate, float *ws, hipStream_t stream);
hipError_t launch_node_product_vjp(int L, int C, int n, int nu, const float *A, const float *W, const float *G,
                                   float *gA, bool accumulate, hipStream_t stream);
hipError_t launch_edge_tp_vjp2(int L, int C, int64_t E, const float *vec, const float *V, const float *w,
                               const float *G, const float *ggV, const float *ggw, const float *ggvec, float *dV,
                               float *dw, float *dr, float *dG, bool accumulate, hipStream_t stream)
{
    ETP_BY_L(edge_tp_vjp2_l, C, E, vec, V, w, G, ggV, ggw, ggvec, dV, dw, dr, dG, accumulate, stream)
}
hipError_t launch_forces(int n_dst, int n_src, const int *row_ptr, const int *src_ptr, const int *perm,
                         const float *gr, float *F, bool accumulate, hipStream_t stream);
size_t transpose_workspace_bytes(int n_src);
hipError_t launch_transpose(int n_dst, int n_src, int64_t E, const int *row_ptr, const int *src, int *src_ptr,
                            int *perm, int *perm_dst, void *ws, hipStream_t stream);
int transpose_noalloc_max_sources();
hipError_t launch_transpose_noalloc(int n_dst, int n_src, int64_t E, const int *row_ptr, const int *src,
                                    int *src_ptr, int *perm, int *perm_dst, hipStream_t stream);
size_t neighbor_workspace_bytes(int n, const float *box, float rc);
size_t block_sum_tmp_floats(int total);
hipError_t launch_block_sum(int64_t n, int64_t stride, int total, const float *part, float *tmp, float *out,
                            bool accumulate, hipStream_t stream);
hipError_t launch_neighbor_count(int n, const float *pos, const float *box, float rc, int *row_ptr, void *ws,
                                 hipStream_t stream);
hipError_t launch_neighbor_fill(int n, const float *pos, const float *box, float rc, const int *row_ptr,
                                int64_t n_edges, int *src, float *vec, void *ws, int **bad, hipStream_t stream);
hipError_t launch_validate(int n_dst, int n_src, int64_t E, const int *row_ptr, const int *src, int *bad,
                           hipStream_t stream);

// the destination-side backward, one translation unit per (l_max, dtype, mode)
#define ETP_DECLARE_BWD(L, XT, MODE) \
    hipError_t ETP_RUN_NAME(bwd, L, XT, MODE)(const ConvArgs &a, float *part, int64_t n_edges, float *grws);
#define ETP_DECLARE_BWD_L(L) \
    ETP_DECLARE_BWD(L, 0, 0) ETP_DECLARE_BWD(L, 0, 1) ETP_DECLARE_BWD(L, 1, 0) ETP_DECLARE_BWD(L, 1, 1)
ETP_DECLARE_BWD_L(0) ETP_DECLARE_BWD_L(1) ETP_DECLARE_BWD_L(2) ETP_DECLARE_BWD_L(3) ETP_DECLARE_BWD_L(4)

const Table *table_for(int L)
{
    switch (L) {
    case 0: return &kTab<0>;
    case 1: return &kTab<1>;
    case 2: return &kTab<2>;
    case 3: return &kTab<3>;
    case 4: return &kTab<4>;
    default: return nullptr;
    }
}

}  // namespace etp

struct etp_plan_s {
    int L, C, dtype;
    const etp::Table *T;
};

namespace {

constexpr int64_t kMaxEdges = 0x7FFFFFFF;

etp_status hip_status(hipError_t e) { return e == hipSuccess ? ETP_OK : ETP_ERR_HIP; }

etp_status check_graph(const etp_graph *g, bool need_transpose)
{
    if (!g)
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_dst < 0 || g->n_src < 0 || g->n_edges < 0)
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_edges >= kMaxEdges)
        return ETP_ERR_UNSUPPORTED;
    if (g->n_dst > 0 && !g->row_ptr)
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_edges > 0 && (!g->src || g->n_src == 0 || g->n_dst == 0))
        return ETP_ERR_INVALID_ARGUMENT;
    if (need_transpose) {
        if (g->n_src > 0 && !g->src_ptr)
            return ETP_ERR_INVALID_ARGUMENT;
        if (g->n_edges > 0 && (!g->perm || !g->perm_dst))
            return ETP_ERR_INVALID_ARGUMENT;
    }
    return ETP_OK;
}

// ETP_FLAG_VALIDATE: count CSR violations on the device (allocates one int
// and synchronises the stream).
etp_status validate_graph(const etp_graph *g, hipStream_t stream)
{
    if (g->n_dst == 0)
        return g->n_edges == 0 ? ETP_OK : ETP_ERR_INTERNAL;
    int *bad = nullptr;
    if (hipMalloc(&bad, sizeof(int)) != hipSuccess)
        return ETP_ERR_ALLOC;
    int host = 0;
    etp_status st = ETP_OK;
    if (hipMemsetAsync(bad, 0, sizeof(int), stream) != hipSuccess ||
        etp::launch_validate(g->n_dst, g->n_src, g->n_edges, g->row_ptr, g->src, bad, stream) != hipSuccess ||
        hipMemcpyAsync(&host, bad, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        st = ETP_ERR_HIP;
    (void)hipFree(bad);
    if (st == ETP_OK && host != 0)
        st = ETP_ERR_INTERNAL;
    return st;
}

#define ETP_RUN_CASES(kind, L, XT)                                                      \
    case (L * 4 + XT * 2 + 0): return etp::ETP_RUN_NAME(kind, L, XT, 0)(a);              \
    case (L * 4 + XT * 2 + 1): return etp::ETP_RUN_NAME(kind, L, XT, 1)(a);

hipError_t run_dst(int L, bool bf16, int mode, const etp::ConvArgs &a)
{
    switch (L * 4 + (bf16 ? 2 : 0) + mode) {
        ETP_RUN_CASES(dst, 0, 0) ETP_RUN_CASES(dst, 0, 1) ETP_RUN_CASES(dst, 1, 0) ETP_RUN_CASES(dst, 1, 1)
        ETP_RUN_CASES(dst, 2, 0) ETP_RUN_CASES(dst, 2, 1) ETP_RUN_CASES(dst, 3, 0) ETP_RUN_CASES(dst, 3, 1)
        ETP_RUN_CASES(dst, 4, 0) ETP_RUN_CASES(dst, 4, 1)
    default: return hipErrorInvalidValue;
    }
}

static_assert(etp::kRadialMax == ETP_MAX_RADIAL_BASIS, "radial basis bound differs from the header's");

hipError_t run_dst_radial(int L, bool bf16, const etp::ConvArgs &a)
{
    switch (L * 2 + (bf16 ? 1 : 0)) {
    case 0: return etp::ETP_RUN_NAME(dst, 0, 0, 2)(a);
    case 1: return etp::ETP_RUN_NAME(dst, 0, 1, 2)(a);
    case 2: return etp::ETP_RUN_NAME(dst, 1, 0, 2)(a);
    case 3: return etp::ETP_RUN_NAME(dst, 1, 1, 2)(a);
    case 4: return etp::ETP_RUN_NAME(dst, 2, 0, 2)(a);
    case 5: return etp::ETP_RUN_NAME(dst, 2, 1, 2)(a);
    case 6: return etp::ETP_RUN_NAME(dst, 3, 0, 2)(a);
    case 7: return etp::ETP_RUN_NAME(dst, 3, 1, 2)(a);
    case 8: return etp::ETP_RUN_NAME(dst, 4, 0, 2)(a);
    case 9: return etp::ETP_RUN_NAME(dst, 4, 1, 2)(a);
    default: return hipErrorInvalidValue;
    }
}

hipError_t run_src_radial(int L, bool bf16, const etp::ConvArgs &a)
{
    switch (L * 2 + (bf16 ? 1 : 0)) {
    case 0: return etp::ETP_RUN_NAME(src, 0, 0, 2)(a);
    case 1: return etp::ETP_RUN_NAME(src, 0, 1, 2)(a);
    case 2: return etp::ETP_RUN_NAME(src, 1, 0, 2)(a);
    case 3: return etp::ETP_RUN_NAME(src, 1, 1, 2)(a);
    case 4: return etp::ETP_RUN_NAME(src, 2, 0, 2)(a);
    case 5: return etp::ETP_RUN_NAME(src, 2, 1, 2)(a);
    case 6: return etp::ETP_RUN_NAME(src, 3, 0, 2)(a);
    case 7: return etp::ETP_RUN_NAME(src, 3, 1, 2)(a);
    case 8: return etp::ETP_RUN_NAME(src, 4, 0, 2)(a);
    case 9: return etp::ETP_RUN_NAME(src, 4, 1, 2)(a);
    default: return hipErrorInvalidValue;
    }
}

// the radial VJP-of-VJP: dG (destination pass) and dx / dh / dr (source pass)
hipError_t run_radial2(bool dst, int L, bool bf16, const etp::ConvArgs &a)
{
#define ETP_RADIAL2_CASE(L)                                                                          \
    case L:                                                                                          \
        if (dst)                                                                                     \
            return bf16 ? etp::ETP_RUN_NAME(dst, L, 1, 3)(a) : etp::ETP_RUN_NAME(dst, L, 0, 3)(a);   \
        return bf16 ? etp::ETP_RUN_NAME(src, L, 1, 3)(a) : etp::ETP_RUN_NAME(src, L, 0, 3)(a);
    switch (L) {
        ETP_RADIAL2_CASE(0) ETP_RADIAL2_CASE(1) ETP_RADIAL2_CASE(2) ETP_RADIAL2_CASE(3) ETP_RADIAL2_CASE(4)
    default: return hipErrorInvalidValue;
    }
#undef ETP_RADIAL2_CASE
}

// the radial source passes that also store weight-gradient partials (modes 4, 5)
hipError_t run_src_wgrad(int L, bool bf16, bool vjp2, const etp::ConvArgs &a)
{
#define ETP_WG_CASE(L)                                                                                 \
    case L:                                                                                            \
        if (vjp2)                                                                                      \
            return bf16 ? etp::ETP_RUN_NAME(src, L, 1, 5)(a) : etp::ETP_RUN_NAME(src, L, 0, 5)(a);     \
        return bf16 ? etp::ETP_RUN_NAME(src, L, 1, 4)(a) : etp::ETP_RUN_NAME(src, L, 0, 4)(a);
    switch (L) {
        ETP_WG_CASE(0) ETP_WG_CASE(1) ETP_WG_CASE(2) ETP_WG_CASE(3) ETP_WG_CASE(4)
    default: return hipErrorInvalidValue;
    }
#undef ETP_WG_CASE
}

// Workspace of the radial weight gradient: per-source-node partials
// [n_src][8][P][C] and the ordered sum's 64 runs [64][8 P C].
size_t wgrad_workspace_bytes(const etp_plan_s *plan, int32_t n_src)
{
    const size_t blk = static_cast<size_t>(ETP_MAX_RADIAL_BASIS) * plan->T->P * plan->C;
    return sizeof(float) * (static_cast<size_t>(n_src) * blk + etp::block_sum_tmp_floats(static_cast<int>(blk)));
}

hipError_t run_src(int L, bool bf16, int mode, const etp::ConvArgs &a)
{
    switch (L * 4 + (bf16 ? 2 : 0) + mode) {
        ETP_RUN_CASES(src, 0, 0) ETP_RUN_CASES(src, 0, 1) ETP_RUN_CASES(src, 1, 0) ETP_RUN_CASES(src, 1, 1)
        ETP_RUN_CASES(src, 2, 0) ETP_RUN_CASES(src, 2, 1) ETP_RUN_CASES(src, 3, 0) ETP_RUN_CASES(src, 3, 1)
        ETP_RUN_CASES(src, 4, 0) ETP_RUN_CASES(src, 4, 1)
    default: return hipErrorInvalidValue;
    }
}

#define ETP_BWD_CASES(L, XT)                                                                 \
    case (L * 4 + XT * 2 + 0): return etp::ETP_RUN_NAME(bwd, L, XT, 0)(a, part, n_edges, grws); \
    case (L * 4 + XT * 2 + 1): return etp::ETP_RUN_NAME(bwd, L, XT, 1)(a, part, n_edges, grws);

hipError_t run_bwd(int L, bool bf16, int mode, const etp::ConvArgs &a, float *part, int64_t n_edges, float *grws)
{
    switch (L * 4 + (bf16 ? 2 : 0) + mode) {
        ETP_BWD_CASES(0, 0) ETP_BWD_CASES(0, 1) ETP_BWD_CASES(1, 0) ETP_BWD_CASES(1, 1) ETP_BWD_CASES(2, 0)
        ETP_BWD_CASES(2, 1) ETP_BWD_CASES(3, 0) ETP_BWD_CASES(3, 1) ETP_BWD_CASES(4, 0) ETP_BWD_CASES(4, 1)
    default: return hipErrorInvalidValue;
    }
}

// Which formulation the workspace entry points use when the caller does not
// force one: the destination-side pass (G rows held per node, node gradient
// through the workspace) where it measured faster on MI355X -- l_max = 3,
// and the l_max = 2 VJP with more than 64 channels -- the source-side pass
// elsewhere (at l_max = 4 the destination side's path groups are too small
// to pay for their repeated edge walks; at l_max <= 2 the source side's G
// rows are few).
bool bwd_uses_dst(int L, int C, bool vjp2, uint32_t flags)
{
    if (flags & ETP_FLAG_DST_PASS)
        return true;
    if (flags & ETP_FLAG_SRC_PASS)
        return false;
    if (vjp2)
        return L == 3;
    return L == 3 || (L == 2 && C > 64);
}

// Workspace of the destination-side backward: one Din-row block per edge,
// then kBwdGrSlices gr / dr partials per edge.
size_t bwd_workspace_bytes(const etp_plan_s *plan, int64_t n_edges)
{
    return static_cast<size_t>(n_edges) * (plan->T->din_rows * plan->C + 3 * etp::kBwdGrSlices) * sizeof(float);
}

// The part rows (when the node gradient is wanted) and the gr / dr partial
// slices (when the workspace is there and large enough) inside ws.
void bwd_split_ws(const etp_plan_s *plan, int64_t n_edges, bool want_x, void *ws, size_t ws_bytes, float **part,
                  float **grws)
{
    const bool whole = ws && (reinterpret_cast<uintptr_t>(ws) & 15u) == 0 && ws_bytes >= bwd_workspace_bytes(plan, n_edges);
    *part = want_x ? static_cast<float *>(ws) : nullptr;
    *grws = whole ? static_cast<float *>(ws) + static_cast<size_t>(n_edges) * plan->T->din_rows * plan->C : nullptr;
}

// box: three finite sides, each at least twice the finite, positive cutoff
etp_status check_neighbor_args(int32_t n, const float *box, float cutoff)
{
    if (n < 0 || !box || !(cutoff > 0.f) || !std::isfinite(cutoff))
        return ETP_ERR_INVALID_ARGUMENT;
    for (int a = 0; a < 3; ++a)
        if (!std::isfinite(box[a]) || !(box[a] > 0.f))
            return ETP_ERR_INVALID_ARGUMENT;
    for (int a = 0; a < 3; ++a)
        if (!(box[a] >= 2.f * cutoff))
            return ETP_ERR_UNSUPPORTED;
    return ETP_OK;
}

}  // namespace

extern "C" {

etp_status etp_plan_create(const etp_plan_desc *desc, etp_plan_t *plan)
{
    if (!desc || !plan)
        return ETP_ERR_INVALID_ARGUMENT;
    *plan = nullptr;
    const int L = desc->l_max_in;
    for (int l : {desc->l_max_in, desc->l_max_sh, desc->l_max_out})
        if (l < 0 || l > etp::kLMax)
            return ETP_ERR_INVALID_ARGUMENT;
    if (desc->channels < 1 || desc->channels > 1024)
        return ETP_ERR_INVALID_ARGUMENT;
    if (desc->x_dtype != ETP_F32 && desc->x_dtype != ETP_BF16)
        return ETP_ERR_INVALID_ARGUMENT;
    if (desc->l_max_sh != L || desc->l_max_out != L)
        return ETP_ERR_UNSUPPORTED;
    if (desc->channels > 64 && (desc->channels & 1))
        return ETP_ERR_UNSUPPORTED;
    const etp::Table *T = etp::table_for(L);
    if (desc->paths) {
        if (desc->n_paths <= 0)
            return ETP_ERR_INVALID_ARGUMENT;
        for (int p = 0; p < desc->n_paths; ++p) {
            const int l1 = desc->paths[3 * p], l2 = desc->paths[3 * p + 1], l3 = desc->paths[3 * p + 2];
            const int lo = l1 > l2 ? l1 - l2 : l2 - l1;
            if (l1 < 0 || l2 < 0 || l3 < lo || l3 > l1 + l2 || l1 > L || l2 > L || l3 > L)
                return ETP_ERR_INVALID_ARGUMENT;
        }
        if (desc->n_paths != T->P)
            return ETP_ERR_UNSUPPORTED;
        for (int p = 0; p < T->P; ++p)
            if (desc->paths[3 * p] != T->path[p].l1 || desc->paths[3 * p + 1] != T->path[p].l2 ||
                desc->paths[3 * p + 2] != T->path[p].l3)
                return ETP_ERR_UNSUPPORTED;
    } else if (desc->n_paths != 0 && desc->n_paths != T->P) {
        return ETP_ERR_INVALID_ARGUMENT;
    }
    etp_plan_s *p = new (std::nothrow) etp_plan_s;
    if (!p)
        return ETP_ERR_ALLOC;
    p->L = L;
    p->C = desc->channels;
    p->dtype = desc->x_dtype;
    p->T = T;
    *plan = p;
    return ETP_OK;
}

etp_status etp_plan_destroy(etp_plan_t plan)
{
    delete plan;
    return ETP_OK;
}

etp_status etp_plan_info(etp_plan_t plan, int32_t *n_paths, int64_t *din, int64_t *dsh, int64_t *dout,
                         int32_t *nnz)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    const etp::Table &T = *plan->T;
    if (n_paths)
        *n_paths = T.P;
    if (din)
        *din = static_cast<int64_t>(plan->C) * T.din_rows;
    if (dsh)
        *dsh = T.dsh;
    if (dout)
        *dout = static_cast<int64_t>(plan->C) * T.dout_rows;
    if (nnz)
        *nnz = T.nnz;
    return ETP_OK;
}

etp_status etp_plan_describe(etp_plan_t plan, etp_plan_info_t *info)
{
    if (!plan || !info)
        return ETP_ERR_INVALID_ARGUMENT;
    info->l_max = plan->L;
    info->channels = plan->C;
    info->x_dtype = plan->dtype;
    info->n_paths = plan->T->P;
    info->nnz = plan->T->nnz;
    info->din_rows = plan->T->din_rows;
    info->dsh = plan->T->dsh;
    info->dout_rows = plan->T->dout_rows;
    return ETP_OK;
}

etp_status etp_plan_tables(etp_plan_t plan, int32_t *paths, int32_t *out_off, int32_t *cg_ptr, int8_t *cg_m,
                           float *cg_val)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    const etp::Table &T = *plan->T;
    for (int p = 0; p < T.P; ++p) {
        if (paths) {
            paths[3 * p] = T.path[p].l1;
            paths[3 * p + 1] = T.path[p].l2;
            paths[3 * p + 2] = T.path[p].l3;
        }
        if (out_off)
            out_off[p] = T.path[p].out_row;
        if (cg_ptr)
            cg_ptr[p] = T.path[p].nz0;
    }
    if (out_off)
        out_off[T.P] = T.dout_rows;
    if (cg_ptr)
        cg_ptr[T.P] = T.nnz;
    for (int t = 0; t < T.nnz; ++t) {
        if (cg_m) {
            cg_m[3 * t] = static_cast<int8_t>(T.nz[t].m1);
            cg_m[3 * t + 1] = static_cast<int8_t>(T.nz[t].m2);
            cg_m[3 * t + 2] = static_cast<int8_t>(T.nz[t].m3);
        }
        if (cg_val)
            cg_val[t] = T.nz[t].fval;
    }
    return ETP_OK;
}

etp_status etp_csr_transpose_workspace(int32_t n_src, size_t *bytes)
{
    if (!bytes || n_src < 0)
        return ETP_ERR_INVALID_ARGUMENT;
    *bytes = etp::transpose_workspace_bytes(n_src);
    return ETP_OK;
}

etp_status etp_workspace_size(etp_plan_t plan, int32_t op, const etp_graph *g, size_t *bytes)
{
    if (!plan || !g || !bytes)
        return ETP_ERR_INVALID_ARGUMENT;
    // a size query reads only the counts: the descriptor's pointers may be NULL
    if (g->n_dst < 0 || g->n_src < 0 || g->n_edges < 0)
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_edges >= kMaxEdges)
        return ETP_ERR_UNSUPPORTED;
    switch (op) {
    case ETP_OP_FWD:
    case ETP_OP_VJP:
    case ETP_OP_VJP2:
        *bytes = 0;  // the convolution keeps everything in registers and LDS
        return ETP_OK;
    case ETP_OP_TRANSPOSE:
        *bytes = etp::transpose_workspace_bytes(g->n_src);
        return ETP_OK;
    case ETP_OP_VJP_WS:
    case ETP_OP_VJP2_WS:
        *bytes = bwd_workspace_bytes(plan, g->n_edges);
        return ETP_OK;
    case ETP_OP_RADIAL_WGRAD:
        *bytes = wgrad_workspace_bytes(plan, g->n_src);
        return ETP_OK;
    case ETP_OP_MIX_WGRAD:
        *bytes = etp::mix_wgrad_workspace_bytes(plan->L, plan->C, g->n_dst);
        return ETP_OK;
    default:
        return ETP_ERR_INVALID_ARGUMENT;
    }
}

etp_status etp_csr_transpose(const etp_graph *g, int32_t *src_ptr, int32_t *perm, int32_t *perm_dst, void *ws,
                             size_t ws_bytes, void *stream)
{
    etp_status st = check_graph(g, false);
    if (st != ETP_OK)
        return st;
    if (!src_ptr || (g->n_edges > 0 && (!perm || !perm_dst)))
        return ETP_ERR_INVALID_ARGUMENT;
    if (!ws || ws_bytes < etp::transpose_workspace_bytes(g->n_src))
        return ETP_ERR_WORKSPACE;
    return hip_status(etp::launch_transpose(g->n_dst, g->n_src, g->n_edges, g->row_ptr, g->src, src_ptr, perm,
                                            perm_dst, ws, static_cast<hipStream_t>(stream)));
}

etp_status etp_csr_transpose_noalloc(const etp_graph *g, int32_t *src_ptr, int32_t *perm, int32_t *perm_dst,
                                     void *stream)
{
    etp_status st = check_graph(g, false);
    if (st != ETP_OK)
        return st;
    if (!src_ptr || (g->n_edges > 0 && (!perm || !perm_dst)))
        return ETP_ERR_INVALID_ARGUMENT;
    static_assert(ETP_NOALLOC_MAX_SOURCES == (1 << 20), "the header's bound differs from the library's");
    if (g->n_src > etp::transpose_noalloc_max_sources())
        return ETP_ERR_WORKSPACE;
    return hip_status(etp::launch_transpose_noalloc(g->n_dst, g->n_src, g->n_edges, g->row_ptr, g->src, src_ptr,
                                                    perm, perm_dst, static_cast<hipStream_t>(stream)));
}

etp_status etp_sh(etp_plan_t plan, int64_t n_edges, const float *vec, float *Y, float *dY, void *stream)
{
    if (!plan || n_edges < 0)
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_edges == 0)
        return ETP_OK;
    if (!vec || !Y)
        return ETP_ERR_INVALID_ARGUMENT;
    return hip_status(etp::launch_sh(plan->L, n_edges, vec, Y, dY, static_cast<hipStream_t>(stream)));
}

etp_status etp_edge_conv_fwd(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *w,
                             float *out, uint32_t flags, void *stream)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    etp_status st = check_graph(g, false);
    if (st != ETP_OK)
        return st;
    if (g->n_dst > 0 && !out)
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_edges > 0 && (!vec || !x || !w))
        return ETP_ERR_INVALID_ARGUMENT;
    if (flags & ~3u)
        return ETP_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        st = validate_graph(g, s);
        if (st != ETP_OK)
            return st;
    }
    etp::ConvArgs a{};
    a.C = plan->C;
    a.n_dst = g->n_dst;
    a.n_src = g->n_src;
    a.row_ptr = g->row_ptr;
    a.src = g->src;
    a.vec = vec;
    a.x = x;
    a.w = w;
    a.out = out;
    a.flags = flags & ETP_FLAG_ACCUMULATE;
    a.stream = s;
    return hip_status(run_dst(plan->L, plan->dtype == ETP_BF16, etp::DST_FWD, a));
}

etp_status etp_edge_conv_fwd_radial(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                    const float *h, int32_t n_basis, const float *Wr, float *out, uint32_t flags,
                                    void *stream)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_basis < 1 || n_basis > ETP_MAX_RADIAL_BASIS)
        return ETP_ERR_UNSUPPORTED;
    etp_status st = check_graph(g, false);
    if (st != ETP_OK)
        return st;
    if (g->n_dst > 0 && !out)
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_edges > 0 && (!vec || !x || !h || !Wr))
        return ETP_ERR_INVALID_ARGUMENT;
    if (flags & ~3u)
        return ETP_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        st = validate_graph(g, s);
        if (st != ETP_OK)
            return st;
    }
    etp::ConvArgs a{};
    a.C = plan->C;
    a.n_dst = g->n_dst;
    a.n_src = g->n_src;
    a.row_ptr = g->row_ptr;
    a.src = g->src;
    a.vec = vec;
    a.x = x;
    a.h = h;
    a.wr = Wr;
    a.nbasis = n_basis;
    a.out = out;
    a.flags = flags & ETP_FLAG_ACCUMULATE;
    a.stream = s;
    return hip_status(run_dst_radial(plan->L, plan->dtype == ETP_BF16, a));
}

etp_status etp_edge_conv_vjp(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *w,
                             const float *grad_out, float *grad_x, float *grad_w, float *grad_vec, uint32_t flags,
                             void *stream)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    etp_status st = check_graph(g, true);
    if (st != ETP_OK)
        return st;
    if (plan->C > 256)
        return ETP_ERR_UNSUPPORTED;
    if (flags & ~3u)
        return ETP_ERR_INVALID_ARGUMENT;
    if (!grad_x && !grad_w && !grad_vec)
        return ETP_OK;
    if (g->n_src > 0 && (!x || !grad_out))
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_edges > 0 && (!vec || !w || !grad_out))
        return ETP_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        st = validate_graph(g, s);
        if (st != ETP_OK)
            return st;
    }
    etp::ConvArgs a{};
    a.C = plan->C;
    a.n_dst = g->n_dst;
    a.n_src = g->n_src;
    a.row_ptr = g->row_ptr;
    a.src = g->src;
    a.src_ptr = g->src_ptr;
    a.perm = g->perm;
    a.perm_dst = g->perm_dst;
    a.vec = vec;
    a.x = x;
    a.w = w;
    a.G = grad_out;
    a.ox = grad_x;
    a.ow = grad_w;
    a.ovec = grad_vec;
    a.flags = flags & ETP_FLAG_ACCUMULATE;
    a.stream = s;
    return hip_status(run_src(plan->L, plan->dtype == ETP_BF16, etp::SRC_VJP, a));
}

etp_status etp_edge_conv_vjp_ws(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *w,
                                const float *grad_out, float *grad_x, float *grad_w, float *grad_vec, uint32_t flags,
                                void *ws, size_t ws_bytes, void *stream)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    etp_status st = check_graph(g, grad_x != nullptr);
    if (st != ETP_OK)
        return st;
    if (plan->C > 256)
        return ETP_ERR_UNSUPPORTED;
    if ((flags & ~15u) || (flags & 12u) == 12u)
        return ETP_ERR_INVALID_ARGUMENT;
    if (!grad_x && !grad_w && !grad_vec)
        return ETP_OK;
    if (g->n_edges > 0 && (!vec || !x || !w || !grad_out))
        return ETP_ERR_INVALID_ARGUMENT;
    const bool dst = bwd_uses_dst(plan->L, plan->C, false, flags);
    if (!dst && grad_x && g->n_src > 0 && (!g->src_ptr || (g->n_edges > 0 && (!g->perm || !g->perm_dst))))
        return ETP_ERR_INVALID_ARGUMENT;
    if (dst && grad_x && g->n_edges > 0 &&
        (!ws || ws_bytes < bwd_workspace_bytes(plan, g->n_edges) || (reinterpret_cast<uintptr_t>(ws) & 15u)))
        return ETP_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        st = validate_graph(g, s);
        if (st != ETP_OK)
            return st;
    }
    etp::ConvArgs a{};
    a.C = plan->C;
    a.n_dst = g->n_dst;
    a.n_src = g->n_src;
    a.row_ptr = g->row_ptr;
    a.src = g->src;
    a.src_ptr = g->src_ptr;
    a.perm = g->perm;
    a.perm_dst = g->perm_dst;
    a.vec = vec;
    a.x = x;
    a.w = w;
    a.G = grad_out;
    a.ox = grad_x;
    a.ow = grad_w;
    a.ovec = grad_vec;
    a.flags = flags & ETP_FLAG_ACCUMULATE;
    a.stream = s;
    if (!dst)
        return hip_status(run_src(plan->L, plan->dtype == ETP_BF16, etp::SRC_VJP, a));
    // (with no edges the kernels still write the zero node rows and read no workspace)
    float *part, *grws;
    bwd_split_ws(plan, g->n_edges, grad_x != nullptr, ws, ws_bytes, &part, &grws);
    return hip_status(run_bwd(plan->L, plan->dtype == ETP_BF16, 0, a, part, g->n_edges, grws));
}

etp_status etp_edge_conv_vjp2_ws(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *w,
                                 const float *grad_out, const float *gg_x, const float *gg_w, const float *gg_vec,
                                 float *d_x, float *d_w, float *d_vec, float *d_grad_out, uint32_t flags, void *ws,
                                 size_t ws_bytes, void *stream)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    etp_status st = check_graph(g, d_x != nullptr);
    if (st != ETP_OK)
        return st;
    if (plan->C > 256)
        return ETP_ERR_UNSUPPORTED;
    if ((flags & ~15u) || (flags & 12u) == 12u)
        return ETP_ERR_INVALID_ARGUMENT;
    if (!d_x && !d_w && !d_vec && !d_grad_out)
        return ETP_OK;
    if (g->n_edges > 0 && (!vec || !x || !w))
        return ETP_ERR_INVALID_ARGUMENT;
    if ((d_x || d_w || d_vec) && g->n_edges > 0 && !grad_out)
        return ETP_ERR_INVALID_ARGUMENT;
    const bool dst = bwd_uses_dst(plan->L, plan->C, true, flags);
    if (!dst && (d_x || d_w || d_vec) && g->n_src > 0 &&
        (!g->src_ptr || (g->n_edges > 0 && (!g->perm || !g->perm_dst))))
        return ETP_ERR_INVALID_ARGUMENT;
    if (dst && d_x && g->n_edges > 0 &&
        (!ws || ws_bytes < bwd_workspace_bytes(plan, g->n_edges) || (reinterpret_cast<uintptr_t>(ws) & 15u)))
        return ETP_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        st = validate_graph(g, s);
        if (st != ETP_OK)
            return st;
    }
    etp::ConvArgs a{};
    a.C = plan->C;
    a.n_dst = g->n_dst;
    a.n_src = g->n_src;
    a.row_ptr = g->row_ptr;
    a.src = g->src;
    a.src_ptr = g->src_ptr;
    a.perm = g->perm;
    a.perm_dst = g->perm_dst;
    a.vec = vec;
    a.x = x;
    a.w = w;
    a.G = grad_out;
    a.ggx = gg_x;
    a.ggw = gg_w;
    a.ggvec = gg_vec;
    a.out = d_grad_out;
    a.ox = d_x;
    a.ow = d_w;
    a.ovec = d_vec;
    a.flags = flags & ETP_FLAG_ACCUMULATE;
    a.stream = s;
    const bool bf16 = plan->dtype == ETP_BF16;
    if (d_grad_out) {  // dG: the destination pass (needs no G)
        st = hip_status(run_dst(plan->L, bf16, etp::DST_DG, a));
        if (st != ETP_OK)
            return st;
    }
    if (!d_x && !d_w && !d_vec)
        return ETP_OK;
    if (!dst)
        return hip_status(run_src(plan->L, bf16, etp::SRC_VJP2, a));
    float *part, *grws;
    bwd_split_ws(plan, g->n_edges, d_x != nullptr, ws, ws_bytes, &part, &grws);
    return hip_status(run_bwd(plan->L, bf16, 1, a, part, g->n_edges, grws));
}

// The source pass with weight-gradient partials, then their ordered sum over
// the source nodes into grad_Wr [n_basis][P][C] (added to under ACCUMULATE).
static etp_status wgrad_finish(etp_plan_t plan, const etp_graph *g, int32_t n_basis, float *grad_Wr, uint32_t flags,
                               void *ws, etp::ConvArgs &a, bool vjp2)
{
    const int64_t blk = static_cast<int64_t>(ETP_MAX_RADIAL_BASIS) * plan->T->P * plan->C;
    float *part = static_cast<float *>(ws);
    a.owr = part;
    etp_status st = hip_status(run_src_wgrad(plan->L, plan->dtype == ETP_BF16, vjp2, a));
    if (st != ETP_OK)
        return st;
    const int total = static_cast<int>(static_cast<int64_t>(n_basis) * plan->T->P * plan->C);
    return hip_status(etp::launch_block_sum(g->n_src, blk, total, part, part + g->n_src * blk, grad_Wr,
                                            (flags & ETP_FLAG_ACCUMULATE) != 0, a.stream));
}

static etp_status radial_vjp(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *h,
                             int32_t n_basis, const float *Wr, const float *grad_out, float *grad_x, float *grad_h,
                             float *grad_vec, float *grad_Wr, uint32_t flags, void *ws, size_t ws_bytes,
                             void *stream)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_basis < 1 || n_basis > ETP_MAX_RADIAL_BASIS)
        return ETP_ERR_UNSUPPORTED;
    etp_status st = check_graph(g, true);
    if (st != ETP_OK)
        return st;
    if (plan->C > 256)
        return ETP_ERR_UNSUPPORTED;
    if (flags & ~3u)
        return ETP_ERR_INVALID_ARGUMENT;
    if (!grad_x && !grad_h && !grad_vec && !grad_Wr)
        return ETP_OK;
    if (g->n_src > 0 && (!x || !grad_out))
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_edges > 0 && (!vec || !h || !Wr || !grad_out))
        return ETP_ERR_INVALID_ARGUMENT;
    if (grad_Wr && (!ws || ws_bytes < wgrad_workspace_bytes(plan, g->n_src) ||
                    (reinterpret_cast<uintptr_t>(ws) & 15u)))
        return ETP_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        st = validate_graph(g, s);
        if (st != ETP_OK)
            return st;
    }
    etp::ConvArgs a{};
    a.C = plan->C;
    a.n_dst = g->n_dst;
    a.n_src = g->n_src;
    a.row_ptr = g->row_ptr;
    a.src = g->src;
    a.src_ptr = g->src_ptr;
    a.perm = g->perm;
    a.perm_dst = g->perm_dst;
    a.vec = vec;
    a.x = x;
    a.h = h;
    a.wr = Wr;
    a.nbasis = n_basis;
    a.G = grad_out;
    a.ox = grad_x;
    a.oh = grad_h;
    a.ovec = grad_vec;
    a.flags = flags & ETP_FLAG_ACCUMULATE;
    a.stream = s;
    if (!grad_Wr)
        return hip_status(run_src_radial(plan->L, plan->dtype == ETP_BF16, a));
    return wgrad_finish(plan, g, n_basis, grad_Wr, flags, ws, a, false);
}

etp_status etp_edge_conv_vjp_radial(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                    const float *h, int32_t n_basis, const float *Wr, const float *grad_out,
                                    float *grad_x, float *grad_h, float *grad_vec, uint32_t flags, void *stream)
{
    return radial_vjp(plan, g, vec, x, h, n_basis, Wr, grad_out, grad_x, grad_h, grad_vec, nullptr, flags, nullptr,
                      0, stream);
}

etp_status etp_edge_conv_vjp_radial_wgrad(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                          const float *h, int32_t n_basis, const float *Wr, const float *grad_out,
                                          float *grad_x, float *grad_h, float *grad_vec, float *grad_Wr,
                                          uint32_t flags, void *ws, size_t ws_bytes, void *stream)
{
    return radial_vjp(plan, g, vec, x, h, n_basis, Wr, grad_out, grad_x, grad_h, grad_vec, grad_Wr, flags, ws,
                      ws_bytes, stream);
}

static etp_status radial_vjp2(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *h,
                              int32_t n_basis, const float *Wr, const float *grad_out, const float *gg_x,
                              const float *gg_h, const float *gg_vec, float *d_x, float *d_h, float *d_vec,
                              float *d_grad_out, float *d_Wr, uint32_t flags, void *ws, size_t ws_bytes,
                              void *stream)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_basis < 1 || n_basis > ETP_MAX_RADIAL_BASIS)
        return ETP_ERR_UNSUPPORTED;
    etp_status st = check_graph(g, true);
    if (st != ETP_OK)
        return st;
    if (plan->C > 256)
        return ETP_ERR_UNSUPPORTED;
    if (flags & ~3u)
        return ETP_ERR_INVALID_ARGUMENT;
    if (!d_x && !d_h && !d_vec && !d_grad_out && !d_Wr)
        return ETP_OK;
    if (g->n_edges > 0 && (!vec || !x || !h || !Wr))
        return ETP_ERR_INVALID_ARGUMENT;
    if ((d_x || d_h || d_vec || d_Wr) && g->n_edges > 0 && !grad_out)
        return ETP_ERR_INVALID_ARGUMENT;
    if (d_Wr && (!ws || ws_bytes < wgrad_workspace_bytes(plan, g->n_src) || (reinterpret_cast<uintptr_t>(ws) & 15u)))
        return ETP_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        st = validate_graph(g, s);
        if (st != ETP_OK)
            return st;
    }
    etp::ConvArgs a{};
    a.C = plan->C;
    a.n_dst = g->n_dst;
    a.n_src = g->n_src;
    a.row_ptr = g->row_ptr;
    a.src = g->src;
    a.src_ptr = g->src_ptr;
    a.perm = g->perm;
    a.perm_dst = g->perm_dst;
    a.vec = vec;
    a.x = x;
    a.h = h;
    a.wr = Wr;
    a.nbasis = n_basis;
    a.G = grad_out;
    a.ggx = gg_x;
    a.ggh = gg_h;
    a.ggvec = gg_vec;
    a.out = d_grad_out;
    a.ox = d_x;
    a.oh = d_h;
    a.ovec = d_vec;
    a.flags = flags & ETP_FLAG_ACCUMULATE;
    a.stream = s;
    const bool bf16 = plan->dtype == ETP_BF16;
    if (d_grad_out) {
        st = hip_status(run_radial2(true, plan->L, bf16, a));
        if (st != ETP_OK)
            return st;
    }
    if (d_Wr)
        return wgrad_finish(plan, g, n_basis, d_Wr, flags, ws, a, true);
    if (d_x || d_h || d_vec)
        return hip_status(run_radial2(false, plan->L, bf16, a));
    return ETP_OK;
}

etp_status etp_edge_conv_vjp2_radial(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                     const float *h, int32_t n_basis, const float *Wr, const float *grad_out,
                                     const float *gg_x, const float *gg_h, const float *gg_vec, float *d_x, float *d_h,
                                     float *d_vec, float *d_grad_out, uint32_t flags, void *stream)
{
    return radial_vjp2(plan, g, vec, x, h, n_basis, Wr, grad_out, gg_x, gg_h, gg_vec, d_x, d_h, d_vec, d_grad_out,
                       nullptr, flags, nullptr, 0, stream);
}

etp_status etp_edge_conv_vjp2_radial_wgrad(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                           const float *h, int32_t n_basis, const float *Wr, const float *grad_out,
                                           const float *gg_x, const float *gg_h, const float *gg_vec, float *d_x,
                                           float *d_h, float *d_vec, float *d_grad_out, float *d_Wr, uint32_t flags,
                                           void *ws, size_t ws_bytes, void *stream)
{
    return radial_vjp2(plan, g, vec, x, h, n_basis, Wr, grad_out, gg_x, gg_h, gg_vec, d_x, d_h, d_vec, d_grad_out,
                       d_Wr, flags, ws, ws_bytes, stream);
}

etp_status etp_edge_conv_vjp2(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *w,
                              const float *grad_out, const float *gg_x, const float *gg_w, const float *gg_vec,
                              float *d_x, float *d_w, float *d_vec, float *d_grad_out, uint32_t flags, void *stream)
{
    if (!plan)
        return ETP_ERR_INVALID_ARGUMENT;
    etp_status st = check_graph(g, true);
    if (st != ETP_OK)
        return st;
    if (plan->C > 256)
        return ETP_ERR_UNSUPPORTED;
    if (flags & ~3u)
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_edges > 0 && (!vec || !x || !w))
        return ETP_ERR_INVALID_ARGUMENT;
    if ((d_x || d_w || d_vec) && g->n_edges > 0 && !grad_out)
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_src > 0 && d_x && !x)
        return ETP_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        st = validate_graph(g, s);
        if (st != ETP_OK)
            return st;
    }
    etp::ConvArgs a{};
    a.C = plan->C;
    a.n_dst = g->n_dst;
    a.n_src = g->n_src;
    a.row_ptr = g->row_ptr;
    a.src = g->src;
    a.src_ptr = g->src_ptr;
    a.perm = g->perm;
    a.perm_dst = g->perm_dst;
    a.vec = vec;
    a.x = x;
    a.w = w;
    a.G = grad_out;
    a.ggx = gg_x;
    a.ggw = gg_w;
    a.ggvec = gg_vec;
    a.out = d_grad_out;
    a.ox = d_x;
    a.ow = d_w;
    a.ovec = d_vec;
    a.flags = flags & ETP_FLAG_ACCUMULATE;
    a.stream = s;
    const bool bf16 = plan->dtype == ETP_BF16;
    if (d_grad_out) {
        st = hip_status(run_dst(plan->L, bf16, etp::DST_DG, a));
        if (st != ETP_OK)
            return st;
    }
    if (d_x || d_w || d_vec)
        return hip_status(run_src(plan->L, bf16, etp::SRC_VJP2, a));
    return ETP_OK;
}

// Both directions of the mixing: the same checks, then one launch.
static etp_status channel_mix_call(bool vjp, etp_plan_t plan, int32_t n_nodes, const float *A, const void *W,
                                   int32_t w_dtype, float *out, uint32_t flags, void *stream)
{
    if (!plan || n_nodes < 0)
        return ETP_ERR_INVALID_ARGUMENT;
    if (flags & ~static_cast<uint32_t>(ETP_FLAG_ACCUMULATE))
        return ETP_ERR_INVALID_ARGUMENT;
    if (w_dtype != ETP_F32 && w_dtype != ETP_BF16)
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_nodes == 0)
        return ETP_OK;
    if (!A || !W || !out)
        return ETP_ERR_INVALID_ARGUMENT;
    const bool bf = w_dtype == ETP_BF16, acc = (flags & ETP_FLAG_ACCUMULATE) != 0;
    const auto st = static_cast<hipStream_t>(stream);
    return hip_status(vjp ? etp::launch_mix_vjp(plan->L, plan->C, n_nodes, A, W, bf, out, acc, st)
                          : etp::launch_mix(plan->L, plan->C, n_nodes, A, W, bf, out, acc, st));
}

etp_status etp_channel_mix(etp_plan_t plan, int32_t n_nodes, const float *in, const float *W, float *out,
                           uint32_t flags, void *stream)
{
    return channel_mix_call(false, plan, n_nodes, in, W, ETP_F32, out, flags, stream);
}

etp_status etp_channel_mix_ex(etp_plan_t plan, int32_t n_nodes, const float *in, const void *W, int32_t w_dtype,
                              float *out, uint32_t flags, void *stream)
{
    return channel_mix_call(false, plan, n_nodes, in, W, w_dtype, out, flags, stream);
}

etp_status etp_channel_mix_vjp(etp_plan_t plan, int32_t n_nodes, const float *grad_y, const float *W, float *grad_in,
                               uint32_t flags, void *stream)
{
    return channel_mix_call(true, plan, n_nodes, grad_y, W, ETP_F32, grad_in, flags, stream);
}

etp_status etp_channel_mix_vjp_ex(etp_plan_t plan, int32_t n_nodes, const float *grad_y, const void *W,
                                  int32_t w_dtype, float *grad_in, uint32_t flags, void *stream)
{
    return channel_mix_call(true, plan, n_nodes, grad_y, W, w_dtype, grad_in, flags, stream);
}

etp_status etp_channel_mix_wgrad(etp_plan_t plan, int32_t n_nodes, const float *in, const float *grad_y,
                                 float *grad_W, uint32_t flags, void *ws, size_t ws_bytes, void *stream)
{
    if (!plan || n_nodes < 0 || !grad_W)
        return ETP_ERR_INVALID_ARGUMENT;
    if (flags & ~static_cast<uint32_t>(ETP_FLAG_ACCUMULATE))
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_nodes > 0 && (!in || !grad_y))
        return ETP_ERR_INVALID_ARGUMENT;
    if (ws && (reinterpret_cast<uintptr_t>(ws) & 15u))
        return ETP_ERR_WORKSPACE;
    return hip_status(etp::launch_mix_wgrad(plan->L, plan->C, n_nodes, in, grad_y, grad_W,
                                            (flags & ETP_FLAG_ACCUMULATE) != 0, static_cast<float *>(ws),
                                            ws ? ws_bytes : 0, static_cast<hipStream_t>(stream)));
}

etp_status etp_edge_tp_fwd(etp_plan_t plan, int64_t n_edges, const float *vec, const float *V, const float *w,
                           float *out, uint32_t flags, void *stream)
{
    if (!plan || n_edges < 0 || (flags & ~static_cast<uint32_t>(ETP_FLAG_ACCUMULATE)))
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_edges >= kMaxEdges)
        return ETP_ERR_UNSUPPORTED;
    if (plan->dtype != ETP_F32)
        return ETP_ERR_UNSUPPORTED;
    if (n_edges == 0)
        return ETP_OK;
    if (!vec || !V || !w || !out)
        return ETP_ERR_INVALID_ARGUMENT;
    return hip_status(etp::launch_edge_tp_fwd(plan->L, plan->C, n_edges, vec, V, w, out,
                                              flags & ETP_FLAG_ACCUMULATE, static_cast<hipStream_t>(stream)));
}

etp_status etp_edge_tp_vjp(etp_plan_t plan, int64_t n_edges, const float *vec, const float *V, const float *w,
                           const float *grad_out, float *grad_V, float *grad_w, float *grad_vec, uint32_t flags,
                           void *stream)
{
    if (!plan || n_edges < 0 || (flags & ~static_cast<uint32_t>(ETP_FLAG_ACCUMULATE)))
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_edges >= kMaxEdges)
        return ETP_ERR_UNSUPPORTED;
    if (plan->dtype != ETP_F32)
        return ETP_ERR_UNSUPPORTED;
    if (n_edges == 0 || (!grad_V && !grad_w && !grad_vec))
        return ETP_OK;
    if (!vec || !V || !w || !grad_out)
        return ETP_ERR_INVALID_ARGUMENT;
    return hip_status(etp::launch_edge_tp_vjp(plan->L, plan->C, n_edges, vec, V, w, grad_out, grad_V, grad_w,
                                              grad_vec, flags & ETP_FLAG_ACCUMULATE,
                                              static_cast<hipStream_t>(stream)));
}

etp_status etp_edge_tp_vjp2(etp_plan_t plan, int64_t n_edges, const float *vec, const float *V, const float *w,
                            const float *grad_out, const float *gg_V, const float *gg_w, const float *gg_vec, float *d_V,
                            float *d_w, float *d_vec, float *d_grad_out, uint32_t flags, void *stream)
{
    if (!plan || n_edges < 0 || (flags & ~static_cast<uint32_t>(ETP_FLAG_ACCUMULATE)))
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_edges >= kMaxEdges)
        return ETP_ERR_UNSUPPORTED;
    if (plan->dtype != ETP_F32)
        return ETP_ERR_UNSUPPORTED;
    if (n_edges == 0 || (!d_V && !d_w && !d_vec && !d_grad_out))
        return ETP_OK;
    if (!vec || !V || !w || !grad_out)
        return ETP_ERR_INVALID_ARGUMENT;
    return hip_status(etp::launch_edge_tp_vjp2(plan->L, plan->C, n_edges, vec, V, w, grad_out, gg_V, gg_w, gg_vec,
                                               d_V, d_w, d_vec, d_grad_out, flags & ETP_FLAG_ACCUMULATE,
                                               static_cast<hipStream_t>(stream)));
}

etp_status etp_node_product(etp_plan_t plan, int32_t n_nodes, int32_t corr_order, const float *A, const float *W,
                            float *out, uint32_t flags, void *stream)
{
    if (!plan || n_nodes < 0 || corr_order < 1 || corr_order > 8)
        return ETP_ERR_INVALID_ARGUMENT;
    if (flags & ~static_cast<uint32_t>(ETP_FLAG_ACCUMULATE))
        return ETP_ERR_INVALID_ARGUMENT;
    if (plan->dtype != ETP_F32)
        return ETP_ERR_UNSUPPORTED;
    if (n_nodes == 0)
        return ETP_OK;
    if (!A || !out || (corr_order > 1 && !W))
        return ETP_ERR_INVALID_ARGUMENT;
    return hip_status(etp::launch_node_product(plan->L, plan->C, n_nodes, corr_order, A, W, out,
                                               flags & ETP_FLAG_ACCUMULATE, static_cast<hipStream_t>(stream)));
}

etp_status etp_node_product_vjp(etp_plan_t plan, int32_t n_nodes, int32_t corr_order, const float *A, const float *W,
                                const float *grad_out, float *grad_A, uint32_t flags, void *stream)
{
    if (!plan || n_nodes < 0 || corr_order < 1 || corr_order > 8)
        return ETP_ERR_INVALID_ARGUMENT;
    if (flags & ~static_cast<uint32_t>(ETP_FLAG_ACCUMULATE))
        return ETP_ERR_INVALID_ARGUMENT;
    if (plan->dtype != ETP_F32)
        return ETP_ERR_UNSUPPORTED;
    if (n_nodes == 0)
        return ETP_OK;
    if (!A || !grad_out || !grad_A || (corr_order > 1 && !W))
        return ETP_ERR_INVALID_ARGUMENT;
    return hip_status(etp::launch_node_product_vjp(plan->L, plan->C, n_nodes, corr_order, A, W, grad_out, grad_A,
                                                   flags & ETP_FLAG_ACCUMULATE, static_cast<hipStream_t>(stream)));
}

etp_status etp_node_product_wgrad_workspace(etp_plan_t plan, int32_t n_nodes, int32_t corr_order, size_t *bytes)
{
    if (!plan || !bytes || n_nodes < 0 || corr_order < 2 || corr_order > 8)
        return ETP_ERR_INVALID_ARGUMENT;
    *bytes = etp::node_product_wgrad_workspace_bytes(plan->L, plan->C, n_nodes, corr_order);
    return ETP_OK;
}

etp_status etp_node_product_vjp_wgrad(etp_plan_t plan, int32_t n_nodes, int32_t corr_order, const float *A,
                                      const float *W, const float *grad_out, float *grad_A, float *grad_W,
                                      uint32_t flags, void *ws, size_t ws_bytes, void *stream)
{
    if (!plan || n_nodes < 0 || corr_order < 2 || corr_order > 8 || !grad_W)
        return ETP_ERR_INVALID_ARGUMENT;
    if (flags & ~static_cast<uint32_t>(ETP_FLAG_ACCUMULATE))
        return ETP_ERR_INVALID_ARGUMENT;
    if (plan->dtype != ETP_F32)
        return ETP_ERR_UNSUPPORTED;
    if (n_nodes > 0 && (!A || !grad_out || !W))
        return ETP_ERR_INVALID_ARGUMENT;
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 15u) ||
        ws_bytes < etp::node_product_wgrad_workspace_bytes(plan->L, plan->C, n_nodes, corr_order))
        return ETP_ERR_WORKSPACE;
    return hip_status(etp::launch_node_product_wgrad(plan->L, plan->C, n_nodes, corr_order, A, W, grad_out, grad_A,
                                                     grad_W, (flags & ETP_FLAG_ACCUMULATE) != 0,
                                                     static_cast<float *>(ws), static_cast<hipStream_t>(stream)));
}

etp_status etp_edge_forces(const etp_graph *g, const float *grad_vec, float *forces, uint32_t flags, void *stream)
{
    etp_status st = check_graph(g, true);
    if (st != ETP_OK)
        return st;
    if (flags & ~3u)
        return ETP_ERR_INVALID_ARGUMENT;
    const int n = g->n_dst > g->n_src ? g->n_dst : g->n_src;
    if (n > 0 && !forces)
        return ETP_ERR_INVALID_ARGUMENT;
    if (g->n_edges > 0 && !grad_vec)
        return ETP_ERR_INVALID_ARGUMENT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        st = validate_graph(g, s);
        if (st != ETP_OK)
            return st;
    }
    return hip_status(etp::launch_forces(g->n_dst, g->n_src, g->row_ptr, g->src_ptr, g->perm, grad_vec, forces,
                                         flags & ETP_FLAG_ACCUMULATE, s));
}

etp_status etp_neighbor_workspace(int32_t n_atoms, const float *box, float cutoff, size_t *bytes)
{
    etp_status st = check_neighbor_args(n_atoms, box, cutoff);
    if (st != ETP_OK)
        return st;
    if (!bytes)
        return ETP_ERR_INVALID_ARGUMENT;
    *bytes = etp::neighbor_workspace_bytes(n_atoms, box, cutoff);
    return ETP_OK;
}

etp_status etp_neighbor_count(int32_t n_atoms, const float *pos, const float *box, float cutoff, int32_t *row_ptr,
                              void *ws, size_t ws_bytes, void *stream)
{
    etp_status st = check_neighbor_args(n_atoms, box, cutoff);
    if (st != ETP_OK)
        return st;
    if (!row_ptr || (n_atoms > 0 && !pos))
        return ETP_ERR_INVALID_ARGUMENT;
    if (!ws || ws_bytes < etp::neighbor_workspace_bytes(n_atoms, box, cutoff))
        return ETP_ERR_WORKSPACE;
    return hip_status(
        etp::launch_neighbor_count(n_atoms, pos, box, cutoff, row_ptr, ws, static_cast<hipStream_t>(stream)));
}

etp_status etp_neighbor_fill(int32_t n_atoms, const float *pos, const float *box, float cutoff, const int32_t *row_ptr,
                             int64_t n_edges, int32_t *src, float *vec, uint32_t flags, void *ws, size_t ws_bytes,
                             void *stream)
{
    etp_status st = check_neighbor_args(n_atoms, box, cutoff);
    if (st != ETP_OK)
        return st;
    if (n_edges < 0 || flags & ~static_cast<uint32_t>(ETP_FLAG_VALIDATE))
        return ETP_ERR_INVALID_ARGUMENT;
    if (n_edges >= kMaxEdges)
        return ETP_ERR_UNSUPPORTED;
    if (!row_ptr || (n_atoms > 0 && !pos) || (n_edges > 0 && (!src || !vec)))
        return ETP_ERR_INVALID_ARGUMENT;
    if (!ws || ws_bytes < etp::neighbor_workspace_bytes(n_atoms, box, cutoff))
        return ETP_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (flags & ETP_FLAG_VALIDATE) {
        // row_ptr must be a CSR of n_edges entries before anything is written
        etp_graph g{n_atoms, n_atoms, n_edges, row_ptr, nullptr, nullptr, nullptr, nullptr};
        if (n_atoms > 0 && (st = validate_graph(&g, s)) != ETP_OK)
            return st;
        if (n_atoms == 0 && n_edges != 0)
            return ETP_ERR_INTERNAL;
    }
    int *bad = nullptr;
    if (etp::launch_neighbor_fill(n_atoms, pos, box, cutoff, row_ptr, n_edges, src, vec, ws, &bad, s) != hipSuccess)
        return ETP_ERR_HIP;
    if (flags & ETP_FLAG_VALIDATE) {
        int host = 0;
        if (hipMemcpyAsync(&host, bad, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return ETP_ERR_HIP;
        if (host != 0)
            return ETP_ERR_INTERNAL;
    }
    return ETP_OK;
}

const char *etp_status_string(etp_status s)
{
    switch (s) {
    case ETP_OK: return "ok";
    case ETP_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ETP_ERR_UNSUPPORTED: return "unsupported by this implementation";
    case ETP_ERR_WORKSPACE: return "workspace missing or too small";
    case ETP_ERR_HIP: return "HIP runtime error";
    case ETP_ERR_ALLOC: return "allocation failed";
    case ETP_ERR_INTERNAL: return "malformed graph or internal error";
    }
    return "unknown status";
}

int32_t etp_version(void) { return 100; }

}  // extern "C"
