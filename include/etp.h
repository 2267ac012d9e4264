/*
 * etp.h -- C ABI of libetp: the fused edge tensor-product convolution of
 * equivariant interatomic potentials on AMD Instinct MI355X (gfx950).
 *
 * The operation. For every edge i <- j of a destination-sorted CSR graph,
 * the real spherical harmonics Y(r_e) of the bond vector r_e (r_src - r_dst)
 * are coupled with the source node's irrep features x[j] through the sparse
 * real Clebsch-Gordan (Wigner 3-j) coefficients of every path (l1, l2, l3),
 * channel by channel ("uvu": one weight per edge, path and channel), scaled
 * by the per-edge weight and summed into the destination node:
 *
 *   out[i, p, m3, u] = sum_{e in in(i)} w[e, p, u]
 *                      sum_{(m1, m2, m3) in p} C[m1, m2, m3] Y_{l2, m2}(r_e) x[src_e, l1, m1, u]
 *
 * This tensor product with sparse Wigner 3-j coefficients is the costly step
 * named in "High-performance training and inference for deep equivariant
 * interatomic potentials" (review page, section "Proposed method") and in
 * "Machine Learning Interatomic Potentials: Advancing Open-Source
 * Software..." (section on the e3j backend); the edge convolution's forward,
 * VJP and VJP-of-VJP are the three stages measured in "How does FlashCart
 * make equivariant interatomic potentials faster and more accurate?"
 * (section "Generated kernels beat SH baselines at high order"). The pages
 * give no formulas; the conventions below are this library's reading of the
 * textbook definitions:
 *   - paths: every (l1, l2, l3) with |l1-l2| <= l3 <= min(l1+l2, l_max) in
 *     lexicographic order (SO(3), no parity selection);
 *   - CG: Racah's formula (Condon-Shortley phase) turned real by the basis
 *     m'>0: (Y^{-m'} + (-1)^m' Y^{m'})/sqrt2, m'<0: i(Y^{m'} - (-1)^m' Y^{-m'})/sqrt2,
 *     keeping the real part for even l1+l2+l3 and the imaginary part for odd;
 *     stored as float32 (round to nearest);
 *   - SH: real, component-normalised (sum_m Y_lm^2 = 2l+1), m = -l..l, z
 *     polar, evaluated at r/|r| (so 1x1->0 is -a.b/sqrt3 and 1x1->1 is
 *     (a x b)/sqrt2 in (y, z, x) order); a zero vector gives Y = (1, 0, ...)
 *     and zero derivatives;
 *   - no path normalisation; one output block per path (block order = path
 *     order).
 *
 * Around the convolution the library provides the other steps of a force
 * call, each declared below with its own contract: the periodic neighbour
 * list that builds the graph (etp_neighbor_*), the stable transpose
 * (etp_csr_transpose), the per-irrep channel mixing and its VJP
 * (etp_channel_mix*), the node-local correlation product and its VJP
 * (etp_node_product*), the edge-local tensor product with its VJP and
 * VJP-of-VJP (etp_edge_tp_*), and the edge-to-atom force assembly
 * (etp_edge_forces).
 *
 * Layouts (row-major, contiguous, channel fastest):
 *   x[n_src][(l_max+1)^2][C]           row l*l + l + m           (f32 or bf16)
 *   w[n_edges][P][C]                   f32
 *   out, grad_out[n_dst][Dout][C]      row off_p + l3 + m3, off_p = sum_{q<p} (2 l3_q + 1)
 *   vec[n_edges][3]                    f32
 *   Y[n_edges][(l_max+1)^2], dY[n_edges][3][(l_max+1)^2]
 * Gradients have the shape of their primals; every float output is f32.
 *
 * Ownership and memory. Every array argument is a DEVICE pointer owned by
 * the caller, at least 16-byte aligned, except where a comment says HOST.
 * The library allocates device memory only in etp_plan_create (nothing
 * today: its tables are compiled in) and for ETP_FLAG_VALIDATE. Calls are
 * asynchronous on the given stream (a hipStream_t passed as void*, NULL =
 * the null stream) and never synchronise it, except ETP_FLAG_VALIDATE.
 * Outputs must not alias inputs. A NULL optional output is not computed; a
 * NULL cotangent means zero.
 *
 * Errors. Argument validation runs on the host before any launch; on error
 * nothing is launched. Device-side data (row_ptr monotone, src in range) is
 * trusted unless ETP_FLAG_VALIDATE is passed. Launch failures return
 * ETP_ERR_HIP.
 *
 * Limits of this implementation: l_max_in = l_max_sh = l_max_out = L in
 * [0, 4]; all paths (paths == NULL or the full list); channels in [1, 1024],
 * even when above 64; the VJP and VJP-of-VJP need channels <= 256; the graph
 * has fewer than 2^31 edges.
 */
#ifndef ETP_H
#define ETP_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define ETP_API __attribute__((visibility("default")))
#else
#define ETP_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct etp_plan_s *etp_plan_t;

typedef enum {
    ETP_OK = 0,
    ETP_ERR_INVALID_ARGUMENT = 1, /* null required pointer, negative size, out-of-range value */
    ETP_ERR_UNSUPPORTED = 2,      /* valid request outside this implementation's limits */
    ETP_ERR_WORKSPACE = 3,        /* workspace missing or too small */
    ETP_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
    ETP_ERR_ALLOC = 5,            /* host or device allocation failed */
    ETP_ERR_INTERNAL = 6,         /* ETP_FLAG_VALIDATE found a malformed graph */
} etp_status;

typedef enum { ETP_F32 = 0, ETP_BF16 = 1 } etp_dtype;

/* Plan descriptor. paths: HOST int32 [n_paths][3] (l1, l2, l3), or NULL for
 * all paths; only the full list is supported. */
typedef struct {
    int32_t l_max_in, l_max_sh, l_max_out;
    int32_t channels;
    int32_t x_dtype; /* etp_dtype of x */
    int32_t n_paths;
    const int32_t *paths;
} etp_plan_desc;

/* A destination-sorted CSR graph. row_ptr[n_dst+1] (row_ptr[0] = 0,
 * row_ptr[n_dst] = n_edges), src[n_edges] in [0, n_src). The stable
 * transpose (from etp_csr_transpose) is needed by the VJP and VJP-of-VJP:
 * src_ptr[n_src+1], perm[n_edges] = edge ids grouped by source in edge-id
 * order, perm_dst[n_edges] = destination of perm[k]. All DEVICE pointers. */
typedef struct {
    int32_t n_dst, n_src;
    int64_t n_edges;
    const int32_t *row_ptr, *src;
    const int32_t *src_ptr, *perm, *perm_dst;
} etp_graph;

typedef struct {
    int32_t l_max, channels, x_dtype;
    int32_t n_paths;   /* P */
    int32_t nnz;       /* CG entries over all paths */
    int32_t din_rows;  /* (l_max+1)^2: rows of x per node */
    int32_t dsh;       /* (l_max+1)^2: SH per edge */
    int32_t dout_rows; /* sum_p (2 l3_p + 1): rows of out per node */
} etp_plan_info_t;

enum {
    ETP_FLAG_ACCUMULATE = 1u, /* node outputs (out, grad_x, d_x, d_grad_out) are added to, not overwritten */
    ETP_FLAG_VALIDATE = 2u,   /* check the CSR on the device first (allocates and synchronises) */
    ETP_FLAG_DST_PASS = 4u,   /* workspace VJP / VJP-of-VJP: walk each destination's in-edges */
    ETP_FLAG_SRC_PASS = 8u,   /* workspace VJP / VJP-of-VJP: walk each source's out-edges */
};

/* Build a plan for (l_max, channels, x dtype): the path list and the sparse
 * real CG table that every convolution call of the plan uses. The pages'
 * tensor-product kernel keeps the Wigner 3-j coefficients in a compressed
 * sparse form ("High-performance training and inference for deep
 * equivariant interatomic potentials", review page, section "Proposed
 * method"), and the forward, VJP and VJP-of-VJP are separate stages over the
 * same tensor product ("How does FlashCart make equivariant interatomic
 * potentials faster and more accurate?", section "Generated kernels beat SH
 * baselines at high order"); the plan is what they share. desc: HOST. The
 * table is compiled into the library, so nothing is allocated. Host only;
 * immutable after creation and usable from several streams. Errors:
 * INVALID_ARGUMENT (null pointers, l_max outside [0, 4], channels outside
 * [1, 1024], unknown dtype, malformed path list), UNSUPPORTED (unequal l_max,
 * a partial path list, odd channels above 64: a valid request this library
 * does not implement). */
ETP_API etp_status etp_plan_create(const etp_plan_desc *desc, etp_plan_t *plan);
ETP_API etp_status etp_plan_destroy(etp_plan_t plan);

/* Sizes of a plan's tensor product (the same source as etp_plan_create),
 * written through HOST pointers (any may be NULL): n_paths = P; din =
 * C (l_max+1)^2 floats of x per node; dsh = (l_max+1)^2 SH per edge; dout =
 * C sum_p (2 l3_p + 1) floats of out per node; nnz = CG entries over all
 * paths. Errors: INVALID_ARGUMENT (null plan). */
ETP_API etp_status etp_plan_info(etp_plan_t plan, int32_t *n_paths, int64_t *din, int64_t *dsh, int64_t *dout,
                                 int32_t *nnz);
/* The same sizes per channel, with the plan's l_max, channels and dtype, in
 * one HOST struct. Errors: INVALID_ARGUMENT (null pointers). */
ETP_API etp_status etp_plan_describe(etp_plan_t plan, etp_plan_info_t *info);

/* The sparse Wigner 3-j table the plan holds ("High-performance training and
 * inference for deep equivariant interatomic potentials", review page,
 * section "Proposed method": the coefficients in compressed sparse form),
 * for verification: copied into HOST buffers (any may be NULL):
 * paths[P][3], out_off[P+1] (first output row of each path), cg_ptr[P+1]
 * (CG entries of path p are [cg_ptr[p], cg_ptr[p+1])), cg_m[nnz][3] (m1, m2,
 * m3, signed, entries ordered by (m1, m2, m3) within a path), cg_val[nnz]
 * (float32 coefficients). */
ETP_API etp_status etp_plan_tables(etp_plan_t plan, int32_t *paths, int32_t *out_off, int32_t *cg_ptr, int8_t *cg_m,
                           float *cg_val);

/* Device workspace (bytes) that etp_csr_transpose needs for n_src sources
 * (host only; errors: INVALID_ARGUMENT for a null pointer or n_src < 0). */
ETP_API etp_status etp_csr_transpose_workspace(int32_t n_src, size_t *bytes);

/* Stable transpose of g's CSR (row_ptr, src, counts in g) into src_ptr,
 * perm, perm_dst (the transpose fields of g are ignored): the neighbour list
 * the convolution walks ("edges per atom" in "How does FlashCart make
 * equivariant interatomic potentials faster and more accurate?", section on
 * the SPICE-MACE-OFF model) grouped by source, which the source-side sums of
 * the backward need (the aggregation of edge contributions that its section
 * "Cartesian kernels replace SH coupling" names as the cost). Integer work,
 * bit-exact and deterministic: perm lists edge ids grouped by source, each
 * group in increasing edge id. src_ptr: DEVICE int32 [n_src + 1]; perm,
 * perm_dst: DEVICE int32 [n_edges]; ws: DEVICE workspace of at least
 * etp_csr_transpose_workspace(n_src) bytes, contents need not be
 * initialised. perm_dst doubles as scratch during the call. Errors:
 * INVALID_ARGUMENT (malformed graph descriptor, null pointers), UNSUPPORTED
 * (n_edges >= 2^31), WORKSPACE (ws missing or too small), HIP. */
ETP_API etp_status etp_csr_transpose(const etp_graph *g, int32_t *src_ptr, int32_t *perm, int32_t *perm_dst, void *ws,
                             size_t ws_bytes, void *stream);

/* etp_csr_transpose for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same transpose with the same result, its workspace taken
 * from a fixed device array inside the library (one per GPU, held until the
 * process ends, sized for n_src <= ETP_NOALLOC_MAX_SOURCES: 4 MiB) instead of
 * a caller buffer. It allocates nothing and calls no allocating routine; the
 * first call on a device looks up that device's copy of the array, with that
 * device current (the stream must belong to the current device). Every call
 * on a GPU shares its array: calls that overlap on one GPU (other streams,
 * other host threads) race and must be ordered by the caller. Arguments as
 * etp_csr_transpose. Errors: INVALID_ARGUMENT (as etp_csr_transpose),
 * WORKSPACE (n_src above ETP_NOALLOC_MAX_SOURCES; nothing is launched),
 * UNSUPPORTED (n_edges >= 2^31), HIP. */
#define ETP_NOALLOC_MAX_SOURCES (1 << 20)
ETP_API etp_status etp_csr_transpose_noalloc(const etp_graph *g, int32_t *src_ptr, int32_t *perm, int32_t *perm_dst,
                                             void *stream);

/* Device workspace (bytes) that an operation needs on graph g (the calls
 * take caller-owned workspaces so that nothing is allocated inside them; the
 * kernels keep intermediates out of memory where they can: "High-performance
 * training and inference for deep equivariant interatomic potentials",
 * review page, section "Proposed method"): ETP_OP_FWD,
 * ETP_OP_VJP and ETP_OP_VJP2 need none (0: the convolution keeps its
 * intermediates in registers and LDS and takes no workspace argument);
 * ETP_OP_TRANSPOSE needs etp_csr_transpose_workspace(g->n_src);
 * ETP_OP_VJP_WS and ETP_OP_VJP2_WS (etp_edge_conv_vjp_ws / _vjp2_ws) need
 * n_edges * (Din * C + 6) * 4 (one Din-row block of the node gradient per
 * edge, then two three-float partials of the bond-vector gradient per edge);
 * ETP_OP_RADIAL_WGRAD (the radial weight gradients) needs
 * (n_src + 64) * ETP_MAX_RADIAL_BASIS * P * C * 4 (per-source-node partials
 * and the runs of their ordered sum); ETP_OP_MIX_WGRAD
 * (etp_channel_mix_wgrad on g->n_dst nodes) needs S * (number of weights) * 4
 * for the S-way split over nodes it uses (0 when it does not split).
 * Host only; reads only the counts in g (its pointers may be NULL).
 * Errors: INVALID_ARGUMENT (null plan, g or bytes, a negative count, an
 * unknown op), UNSUPPORTED (n_edges >= 2^31). */
enum {
    ETP_OP_FWD = 0,
    ETP_OP_VJP = 1,
    ETP_OP_VJP2 = 2,
    ETP_OP_TRANSPOSE = 3,
    ETP_OP_VJP_WS = 4,
    ETP_OP_VJP2_WS = 5,
    ETP_OP_RADIAL_WGRAD = 6,
    ETP_OP_MIX_WGRAD = 7
};
ETP_API etp_status etp_workspace_size(etp_plan_t plan, int32_t op, const etp_graph *g, size_t *bytes);

/* Real spherical harmonics of n_edges bond vectors, the second operand of the
 * tensor product (the SH coupling of "How does FlashCart make equivariant
 * interatomic potentials faster and more accurate?", section "Cartesian
 * kernels replace SH coupling"; the convolution kernels evaluate them in
 * registers, this call exposes them): Y[n][dsh] and, if dY is not NULL,
 * dY[n][3][dsh] = dY/dr (with respect to the unnormalised vector), in the
 * conventions listed at the top of this file. vec: DEVICE float [n][3]; Y,
 * dY: DEVICE float. Errors: INVALID_ARGUMENT (null plan or pointers with
 * n_edges > 0, n_edges < 0), HIP. */
ETP_API etp_status etp_sh(etp_plan_t plan, int64_t n_edges, const float *vec, float *Y, float *dY, void *stream);

/* Forward: out[n_dst][Dout][C] from vec, x (plan dtype), w. */
ETP_API etp_status etp_edge_conv_fwd(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *w,
                             float *out, uint32_t flags, void *stream);

/* Forward with the per-edge weights formed inside the kernel from the last
 * layer of a radial network instead of read from memory:
 *   w[e, p, u] = sum_{k < n_basis} h[e, k] Wr[(k*P + p)*C + u]
 * then out as in etp_edge_conv_fwd. The pages' kernels keep intermediates
 * out of memory ("High-performance training and inference for deep
 * equivariant interatomic potentials", section "Proposed method") and weight
 * each path by a learned function of the edge's radial features ("Scaling
 * the leading accuracy of deep equivariant models to biomolecular
 * simulations of realistic size", section "Proposed method"); the pages do
 * not fix the network, and this is its linear last layer, whose E*P*C
 * weights would otherwise be the largest stream the forward reads.
 * h:  DEVICE float [n_edges][n_basis] (features after the radial network's
 *     hidden layers and any envelope), 1 <= n_basis <= ETP_MAX_RADIAL_BASIS;
 * Wr: DEVICE float [n_basis][P][C], shared by all edges.
 * Other arguments, layouts and flags as etp_edge_conv_fwd; fp32 sums of
 * n_basis terms in k order. Errors: UNSUPPORTED (n_basis out of range),
 * INVALID_ARGUMENT (null pointers, a malformed graph, unknown flags). */
#define ETP_MAX_RADIAL_BASIS 8
ETP_API etp_status etp_edge_conv_fwd_radial(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                            const float *h, int32_t n_basis, const float *Wr, float *out,
                                            uint32_t flags, void *stream);

/* VJP: given grad_out = dL/dout, grad_x = dL/dx (source-segmented),
 * grad_w = dL/dw and grad_vec = dL/dvec (forces on the edges). Each output
 * may be NULL. Needs the transpose in g. */
ETP_API etp_status etp_edge_conv_vjp(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *w,
                             const float *grad_out, float *grad_x, float *grad_w, float *grad_vec, uint32_t flags,
                             void *stream);

/* The VJP and VJP-of-VJP walked over each destination's in-edges instead of
 * each source's out-edges, for callers that can lend a workspace. The
 * backward's widest operand is the cotangent G[i] (Dout rows per node, several
 * times the Din rows of x), and the pages locate the convolution's cost in
 * memory access and edge aggregation ("How does FlashCart make equivariant
 * interatomic potentials faster and more accurate?", section "Cartesian
 * kernels replace SH coupling"; the VJP and VJP-of-VJP are the stages of its
 * section "Generated kernels beat SH baselines at high order"): here each
 * node's G rows are read once and kept in registers while its in-edges
 * stream w (and W') and gather the x (and X') rows of their sources. The
 * per-edge weight, bond-vector and (VJP-of-VJP) d_grad_out results come out
 * of that pass directly; the node gradient grad_x (d_x) is first written as
 * one Din-row block per edge into ws (ws[e][Din][C] floats) and then summed
 * over each source's out-edges in the order of the stable transpose (fixed
 * order, no atomics: bitwise deterministic). The VJP-of-VJP's d_grad_out
 * comes from the destination pass that etp_edge_conv_vjp2 uses. Where the
 * source-side walk of etp_edge_conv_vjp / _vjp2 measured faster (l_max 0, 1
 * and 4, and the l_max = 2 VJP-of-VJP and VJP with C <= 64) these calls run
 * it instead and leave ws unused; ETP_FLAG_DST_PASS or ETP_FLAG_SRC_PASS
 * forces one formulation (not both). Results equal those of
 * etp_edge_conv_vjp / etp_edge_conv_vjp2 up to rounding order (each
 * formulation is deterministic on its own); arguments, shapes and null
 * conventions are the same.
 * ws: DEVICE workspace, 16-byte aligned, of at least
 * etp_workspace_size(plan, ETP_OP_VJP_WS / ETP_OP_VJP2_WS, g) bytes
 * (n_edges * (Din * C + 6) * 4), needed when grad_x (d_x) is requested from
 * the destination-side formulation; without grad_x it may be NULL, and
 * when given it lets the path groups of l_max = 3 run in one launch (their
 * bond-vector partials are added in group order afterwards: the same
 * result, bit for bit); its contents need not be initialised and are
 * undefined afterwards. The transpose in g is needed for grad_x
 * (d_x), and for every output of the source-side formulation. Errors: as
 * etp_edge_conv_vjp / etp_edge_conv_vjp2, plus WORKSPACE (ws missing,
 * misaligned or too small while grad_x / d_x is requested). */
ETP_API etp_status etp_edge_conv_vjp_ws(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                        const float *w, const float *grad_out, float *grad_x, float *grad_w,
                                        float *grad_vec, uint32_t flags, void *ws, size_t ws_bytes, void *stream);
ETP_API etp_status etp_edge_conv_vjp2_ws(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                         const float *w, const float *grad_out, const float *gg_x,
                                         const float *gg_w, const float *gg_vec, float *d_x, float *d_w,
                                         float *d_vec, float *d_grad_out, uint32_t flags, void *ws, size_t ws_bytes,
                                         void *stream);

/* VJP of etp_edge_conv_fwd_radial (the force call of a model whose path
 * weights come from radial features): with w = h Wr formed in the kernel as
 * in the forward, grad_x and grad_vec as etp_edge_conv_vjp gives them, and
 * instead of grad_w its contraction with the last layer,
 *   grad_h[e, k] = sum_{p,u} grad_w[e, p, u] Wr[(k*P + p)*C + u]
 * (DEVICE float [n_edges][n_basis]; with grad_vec it yields the forces
 * through h's dependence on |r|). Outputs may be NULL; ETP_FLAG_ACCUMULATE
 * applies to grad_x only. Sums over channels,
 * paths and channel chunks are in a fixed order (deterministic). Needs the
 * transpose in g; C <= 256. The gradient with respect to Wr comes from
 * etp_edge_conv_vjp_radial_wgrad. Errors as etp_edge_conv_fwd_radial, plus
 * UNSUPPORTED for C > 256. */
ETP_API etp_status etp_edge_conv_vjp_radial(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                            const float *h, int32_t n_basis, const float *Wr,
                                            const float *grad_out, float *grad_x, float *grad_h, float *grad_vec,
                                            uint32_t flags, void *stream);

/* VJP of etp_edge_conv_vjp_radial (force training of a model whose path
 * weights come from radial features, with no E*P*C weight array in memory:
 * "High-performance training and inference for deep equivariant interatomic
 * potentials", review page, section "Proposed method"; the VJP-of-VJP stage
 * of "How does FlashCart make equivariant interatomic potentials faster and
 * more accurate?", section "Generated kernels beat SH baselines at high
 * order"): with cotangents (gg_x, gg_h, gg_vec) on (grad_x, grad_h, grad_vec),
 * the gradients of S = <gg_x, grad_x> + <gg_h, grad_h> + <gg_vec, grad_vec>
 * with respect to x (d_x), h (d_h, DEVICE float [n_edges][n_basis]), vec
 * (d_vec) and grad_out (d_grad_out). Since grad_h = grad_w Wr, the cotangent
 * gg_h acts as gg_w = gg_h Wr, formed in the kernels like w = h Wr, and the
 * weight cotangent is contracted back, d_h[e, k] = sum_{p,u} d_w[e, p, u]
 * Wr[(k*P + p)*C + u]; the result equals etp_edge_conv_vjp2 with w = h Wr,
 * gg_w = gg_h Wr and d_w contracted with Wr. The gradient with respect to Wr
 * comes from etp_edge_conv_vjp2_radial_wgrad. Cotangents may be NULL (zero); outputs may be NULL.
 * ETP_FLAG_ACCUMULATE applies to d_x and d_grad_out. Sums in a fixed order
 * (deterministic). Needs the transpose in g; C <= 256. Errors as
 * etp_edge_conv_vjp_radial. */
ETP_API etp_status etp_edge_conv_vjp2_radial(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x,
                                             const float *h, int32_t n_basis, const float *Wr, const float *grad_out,
                                             const float *gg_x, const float *gg_h, const float *gg_vec, float *d_x,
                                             float *d_h, float *d_vec, float *d_grad_out, uint32_t flags,
                                             void *stream);

/* The radial VJP and VJP-of-VJP that also form the gradient with respect to
 * the last-layer matrix Wr (training the radial network end to end; the
 * pages weight each path by a learned function of the edge's radial
 * features: "Scaling the leading accuracy of deep equivariant models to
 * biomolecular simulations of realistic size", section "Proposed method"):
 *   etp_edge_conv_vjp_radial_wgrad:  grad_Wr[k, p, u] = sum_e h[e, k] gw[e, p, u]
 *   etp_edge_conv_vjp2_radial_wgrad: d_Wr[k, p, u] = sum_e h[e, k] dw[e, p, u]
 *                                                  + sum_e gg_h[e, k] gw[e, p, u]
 * with gw, dw the per-edge weight cotangents the calls never store (the
 * second term because grad_h = gw Wr depends on Wr). grad_Wr / d_Wr: DEVICE
 * float [n_basis][P][C], the layout of Wr. Every other argument, output and
 * flag as etp_edge_conv_vjp_radial / etp_edge_conv_vjp2_radial, whose results
 * these calls reproduce up to rounding order (their path groups are cut
 * smaller to make room for the partial sums). The sum over
 * edges is formed per source node in the kernels (each lane its channel,
 * the node's edge splits added in a fixed order) into ws, then added over
 * the source nodes in index order by a two-level kernel: deterministic, no
 * atomics. ETP_FLAG_ACCUMULATE also adds into grad_Wr / d_Wr. ws: DEVICE,
 * 16-byte aligned, at least etp_workspace_size(plan, ETP_OP_RADIAL_WGRAD, g)
 * bytes, contents undefined afterwards. Errors: as the calls without the
 * weight gradient, plus WORKSPACE (ws missing, misaligned or too small). */
ETP_API etp_status etp_edge_conv_vjp_radial_wgrad(etp_plan_t plan, const etp_graph *g, const float *vec,
                                                  const void *x, const float *h, int32_t n_basis, const float *Wr,
                                                  const float *grad_out, float *grad_x, float *grad_h,
                                                  float *grad_vec, float *grad_Wr, uint32_t flags, void *ws,
                                                  size_t ws_bytes, void *stream);
ETP_API etp_status etp_edge_conv_vjp2_radial_wgrad(etp_plan_t plan, const etp_graph *g, const float *vec,
                                                   const void *x, const float *h, int32_t n_basis, const float *Wr,
                                                   const float *grad_out, const float *gg_x, const float *gg_h,
                                                   const float *gg_vec, float *d_x, float *d_h, float *d_vec,
                                                   float *d_grad_out, float *d_Wr, uint32_t flags, void *ws,
                                                   size_t ws_bytes, void *stream);

/* VJP of the VJP: with cotangents (gg_x, gg_w, gg_vec) on (grad_x, grad_w,
 * grad_vec), the gradients of S = <gg_x, grad_x> + <gg_w, grad_w> +
 * <gg_vec, grad_vec> with respect to x (d_x), w (d_w), vec (d_vec) and
 * grad_out (d_grad_out). Cotangents may be NULL (zero; gg_x is f32 even for
 * bf16 plans); outputs may be NULL. Needs the transpose in g. */
ETP_API etp_status etp_edge_conv_vjp2(etp_plan_t plan, const etp_graph *g, const float *vec, const void *x, const float *w,
                              const float *grad_out, const float *gg_x, const float *gg_w, const float *gg_vec,
                              float *d_x, float *d_w, float *d_vec, float *d_grad_out, uint32_t flags,
                              void *stream);

/* Per-irrep channel mixing after the convolution (the dense channel
 * contraction that follows the tensor product: "Scaling the leading accuracy
 * of deep equivariant models to biomolecular simulations of realistic size",
 * section "Proposed method"; the pages do not fix its form, and this is one
 * matrix per output order shared by that order's components):
 *   out[i][l*l + m][v] = sum_{p: l3_p = l} sum_u W_l[(q_p*C + u)*C + v] * in[i][off_p + m][u]
 * for i < n_nodes, l = 0..l_max, m < 2l + 1, v < C; q_p is the rank of path p
 * among the paths of order l (path order) and off_p its first output row.
 * in:  DEVICE float [n_nodes][dout_rows][C] (a convolution output);
 * W:   DEVICE float W_0, W_1, ..., W_lmax back to back, W_l of n_l*C rows
 *      and C columns (row-major), n_l = number of paths with l3 = l;
 * out: DEVICE float [n_nodes][(l_max+1)^2][C] (the node-feature layout).
 * fp32 in and out, fp32 matrix-core accumulation. flags: ETP_FLAG_ACCUMULATE
 * adds into out. The caller owns every buffer; nothing is allocated. Errors:
 * INVALID_ARGUMENT (null plan or pointers with n_nodes > 0, negative
 * n_nodes, other flags), HIP (launch failure). */
ETP_API etp_status etp_channel_mix(etp_plan_t plan, int32_t n_nodes, const float *in, const float *W, float *out,
                                   uint32_t flags, void *stream);

/* etp_channel_mix with a choice of weight precision (the pages run the
 * dense contraction after the tensor product in mixed precision: "Scaling
 * the leading accuracy of deep equivariant models to biomolecular
 * simulations of realistic size", section "Proposed method"). W: DEVICE, the
 * layout of etp_channel_mix, in w_dtype: ETP_F32 (fp32 matrix-core products,
 * 16x16x4: the result of etp_channel_mix, bit for bit) or ETP_BF16 (raw
 * bfloat16; the fp32 input is rounded to bf16, nearest even, as it is
 * loaded, and 16x16x32 bf16 matrix-core products accumulate in fp32). in,
 * out and flags as etp_channel_mix; nothing is allocated. Errors:
 * INVALID_ARGUMENT (as etp_channel_mix, or an unknown w_dtype), HIP. */
ETP_API etp_status etp_channel_mix_ex(etp_plan_t plan, int32_t n_nodes, const float *in, const void *W, int32_t w_dtype,
                                      float *out, uint32_t flags, void *stream);

/* VJP of etp_channel_mix with respect to its input (the mixing is linear, so
 * this is the transposed map; forces flow through it):
 *   grad_in[i][off_p + m][u] = sum_v W_l[(q_p*C + u)*C + v] * grad_y[i][l*l + m][v]
 * for every path p of order l = l3_p. grad_y: DEVICE float
 * [n_nodes][(l_max+1)^2][C]; W as for etp_channel_mix; grad_in: DEVICE float
 * [n_nodes][dout_rows][C]. fp32 matrix-core accumulation. The weight gradient
 * (a sum over all nodes) is not computed. flags: ETP_FLAG_ACCUMULATE adds into
 * grad_in. Errors as for etp_channel_mix. */
ETP_API etp_status etp_channel_mix_vjp(etp_plan_t plan, int32_t n_nodes, const float *grad_y, const float *W,
                                       float *grad_in, uint32_t flags, void *stream);

/* etp_channel_mix_vjp with W in w_dtype (ETP_F32: the result of
 * etp_channel_mix_vjp, bit for bit; ETP_BF16: grad_y rounded to bf16 as it
 * is loaded, bf16 matrix-core products, fp32 accumulation), as
 * etp_channel_mix_ex is to etp_channel_mix. Errors as etp_channel_mix_ex. */
ETP_API etp_status etp_channel_mix_vjp_ex(etp_plan_t plan, int32_t n_nodes, const float *grad_y, const void *W,
                                          int32_t w_dtype, float *grad_in, uint32_t flags, void *stream);

/* Gradient of the channel mixing with respect to its weights (training the
 * dense contraction after the tensor product: "Scaling the leading accuracy
 * of deep equivariant models to biomolecular simulations of realistic size",
 * section "Proposed method"):
 *   grad_W_l[(q_p*C + u)*C + v] = sum_{i < n_nodes} sum_{m < 2l+1}
 *                                 in[i][off_p + m][u] * grad_y[i][l*l + m][v]
 * for every path p of order l = l3_p, in the layout of W (etp_channel_mix).
 * in: DEVICE float [n_nodes][dout_rows][C]; grad_y: DEVICE float
 * [n_nodes][(l_max+1)^2][C]; grad_W: DEVICE float, the size of W. fp32
 * matrix-core products (16x16x4), fp32 accumulation; the sum over nodes is
 * split over S workgroups per output tile, whose partial blocks go to ws and
 * are added in split order (deterministic, no atomics). ws: NULL, or a
 * 16-byte aligned DEVICE workspace of etp_workspace_size(plan,
 * ETP_OP_MIX_WGRAD, g with n_dst = n_nodes) bytes; NULL or a smaller one
 * means one workgroup per tile takes every node (same result up to rounding
 * order, slower). flags: ETP_FLAG_ACCUMULATE adds into grad_W; with
 * n_nodes = 0 grad_W is zeroed (or left as it is when accumulating).
 * Errors: INVALID_ARGUMENT (null plan or grad_W, null in / grad_y with
 * n_nodes > 0, negative n_nodes, other flags), WORKSPACE (misaligned ws),
 * HIP. */
ETP_API etp_status etp_channel_mix_wgrad(etp_plan_t plan, int32_t n_nodes, const float *in, const float *grad_y,
                                         float *grad_W, uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* Edge-local tensor product: the convolution's message without the
 * destination sum, one output block per edge (the pair-wise tensor product of
 * Allegro, whose energy is a sum of per-pair terms: "Scaling the leading
 * accuracy of deep equivariant models to biomolecular simulations of
 * realistic size", section "Proposed method"):
 *   out[e][off_p + l3 + m3][u] = w[e][p][u]
 *        sum_{(m1, m2, m3) in p} C[m1, m2, m3] Y_{l2, m2}(vec_e) V[e][l1*l1 + l1 + m1][u]
 * (the forward of the convolution on a graph where every edge is its own
 * destination and source). V: DEVICE float [n_edges][(l_max+1)^2][C];
 * w: [n_edges][P][C]; vec: [n_edges][3]; out, grad_out: [n_edges][dout_rows][C].
 * The VJP gives grad_V, grad_w and grad_vec (each may be NULL: not computed).
 * fp32 only (the plan must be ETP_F32). flags: ETP_FLAG_ACCUMULATE adds into
 * every output. Nothing is allocated; no atomics (deterministic). Errors:
 * INVALID_ARGUMENT (null plan or pointers, negative n_edges, other flags),
 * UNSUPPORTED (bf16 plan, n_edges >= 2^31), HIP. */
ETP_API etp_status etp_edge_tp_fwd(etp_plan_t plan, int64_t n_edges, const float *vec, const float *V, const float *w,
                                   float *out, uint32_t flags, void *stream);
ETP_API etp_status etp_edge_tp_vjp(etp_plan_t plan, int64_t n_edges, const float *vec, const float *V, const float *w,
                                   const float *grad_out, float *grad_V, float *grad_w, float *grad_vec,
                                   uint32_t flags, void *stream);
/* VJP of the edge-local VJP (force training): with cotangents (gg_V, gg_w,
 * gg_vec) on (grad_V, grad_w, grad_vec), the gradients of
 * S = <gg_V, grad_V> + <gg_w, grad_w> + <gg_vec, grad_vec> with respect to V
 * (d_V), w (d_w), vec (d_vec) and grad_out (d_grad_out); the same as
 * etp_edge_conv_vjp2 on the graph where every edge is its own destination
 * and source. Cotangents may be NULL (zero); outputs may be NULL. Shapes and
 * flags as for etp_edge_tp_vjp. */
ETP_API etp_status etp_edge_tp_vjp2(etp_plan_t plan, int64_t n_edges, const float *vec, const float *V,
                                    const float *w, const float *grad_out, const float *gg_V, const float *gg_w,
                                    const float *gg_vec, float *d_V, float *d_w, float *d_vec, float *d_grad_out,
                                    uint32_t flags, void *stream);

/* Node-local correlation product: weighted products of each node's irreps
 * with themselves, applied step by step and truncated to orders <= l_max
 * after every step (the node-local product ladder of "How does FlashCart
 * make equivariant interatomic potentials faster and more accurate?",
 * section "Generated kernels beat SH baselines at high order"; the page
 * gives no formula, this is the channel-wise reading):
 *   B_1 = A,
 *   B_{k+1}[i][l3*l3 + l3 + m3][u] = sum_{p = (l1, l2, l3)} W[k-1][p][u]
 *        sum_{(m1, m2, m3)} C_p[m1, m2, m3] B_k[i][l1 row, m1][u] A[i][l2 row, m2][u],
 *   out = B_1 + ... + B_nu                    (nu = corr_order, in [1, 8])
 * over the plan's paths and real CG table (l1, l2, l3 <= l_max).
 * A, out: DEVICE float [n_nodes][(l_max+1)^2][C]; W: DEVICE float
 * [corr_order-1][P][C] (may be NULL when corr_order is 1). fp32 throughout;
 * the plan must be ETP_F32. flags: ETP_FLAG_ACCUMULATE adds into out. Nothing
 * is allocated. Errors: INVALID_ARGUMENT (null plan or pointers, negative
 * n_nodes, corr_order outside [1, 8], other flags), UNSUPPORTED (a bf16
 * plan), HIP. */
ETP_API etp_status etp_node_product(etp_plan_t plan, int32_t n_nodes, int32_t corr_order, const float *A,
                                    const float *W, float *out, uint32_t flags, void *stream);

/* VJP of etp_node_product with respect to A (what forces need, A being
 * built from the positions): grad_A = d<grad_out, out>/dA, by reverse mode
 * over the ladder with each B_k recomputed from A in registers. grad_out,
 * grad_A: DEVICE float [n_nodes][(l_max+1)^2][C]; the other arguments as in
 * etp_node_product. The weight gradient (a sum over all nodes) is not
 * computed. flags: ETP_FLAG_ACCUMULATE adds into grad_A. Errors as for
 * etp_node_product. */
ETP_API etp_status etp_node_product_vjp(etp_plan_t plan, int32_t n_nodes, int32_t corr_order, const float *A,
                                        const float *W, const float *grad_out, float *grad_A, uint32_t flags,
                                        void *stream);

/* etp_node_product_vjp that also forms the gradient with respect to the
 * weights (training the ladder; a sum over every node):
 *   grad_W[k][p][u] = sum_i d<grad_out, out>/dW[k][p][u]
 *                   = sum_i sum_{(m1, m2, m3) in p} C_p * Bbar_{k+2}[i][l3 row, m3][u]
 *                         * B_{k+1}[i][l1 row, m1][u] * A[i][l2 row, m2][u]
 * (Bbar the adjoints of the reverse pass, k = 0 .. corr_order-2). The
 * reverse pass writes each node's [corr_order-1][P][C] block of partials to
 * ws, and they are added over the nodes in index order (runs of nodes, then
 * the runs in order): deterministic, no atomics. grad_A: as
 * etp_node_product_vjp, or NULL (not computed); grad_W: DEVICE float
 * [corr_order-1][P][C], the layout of W. ETP_FLAG_ACCUMULATE adds into
 * grad_A and grad_W (with n_nodes = 0 grad_W is zeroed, or left as it is when
 * accumulating). ws: DEVICE, 16-byte aligned, at least
 * etp_node_product_wgrad_workspace(plan, n_nodes, corr_order) bytes, contents
 * undefined afterwards. Errors: INVALID_ARGUMENT (null plan or grad_W, null A,
 * W or grad_out with n_nodes > 0, negative n_nodes, corr_order outside
 * [2, 8], other flags), UNSUPPORTED (a bf16 plan), WORKSPACE (ws missing,
 * misaligned or too small), HIP. */
ETP_API etp_status etp_node_product_vjp_wgrad(etp_plan_t plan, int32_t n_nodes, int32_t corr_order, const float *A,
                                              const float *W, const float *grad_out, float *grad_A, float *grad_W,
                                              uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* Workspace (bytes) of etp_node_product_vjp_wgrad: n_nodes * (corr_order-1)
 * * P * C * 4 for the per-node partials plus 64 * (corr_order-1) * P * C * 4
 * for the runs of their ordered sum. Host only. Errors: INVALID_ARGUMENT
 * (null plan or bytes, negative n_nodes, corr_order outside [2, 8]). */
ETP_API etp_status etp_node_product_wgrad_workspace(etp_plan_t plan, int32_t n_nodes, int32_t corr_order,
                                                    size_t *bytes);

/* Forces on the atoms from the per-edge energy gradient grad_vec = dE/dvec
 * (the VJP's grad_vec), with vec_e = pos[src_e] - pos[dst_e]:
 *   forces[k] = sum_{e in in(k)} grad_vec[e] - sum_{e in out(k)} grad_vec[e]
 * for k < max(n_dst, n_src) (energy and forces from one model: "How does
 * FlashCart make equivariant interatomic potentials faster and more
 * accurate?", section on the SPICE-MACE-OFF model). g needs the transpose
 * (src_ptr, perm). grad_vec: DEVICE float [n_edges][3]; forces: DEVICE float
 * [max(n_dst, n_src)][3]. Fixed-order sums, no atomics. flags:
 * ETP_FLAG_ACCUMULATE adds into forces, ETP_FLAG_VALIDATE checks the CSR
 * first. The caller owns every buffer. Errors: INVALID_ARGUMENT (null graph,
 * missing transpose, null pointers, other flags), UNSUPPORTED (n_edges >=
 * 2^31), INTERNAL (malformed graph under VALIDATE), HIP (launch failure). */
ETP_API etp_status etp_edge_forces(const etp_graph *g, const float *grad_vec, float *forces, uint32_t flags,
                                   void *stream);

/* Periodic neighbour list: the destination-sorted CSR graph and bond vectors
 * the convolution walks ("edges per atom" in "How does FlashCart make
 * equivariant interatomic potentials faster and more accurate?", section on
 * the SPICE-MACE-OFF model). For n_atoms atoms at pos (DEVICE float
 * [n_atoms][3]) in an orthorhombic periodic box (box: HOST float[3], every
 * side at least 2 * cutoff), row i lists every j != i with
 *   q = p - L floor(p / L),  d = q_j - q_i,  d = d - L rint(d / L)   (per axis)
 *   fma(dz, dz, fma(dy, dy, dx * dx)) < cutoff * cutoff
 * evaluated in float32 exactly as written (correctly rounded division,
 * round-half-even rint), sources ascending; vec of that edge = d (the
 * minimum image of pos[j] - pos[i]). The edges are therefore bit-exact and
 * deterministic. Two calls, because the edge count is known only on the
 * device:
 *   1. etp_neighbor_count writes row_ptr (DEVICE int32 [n_atoms + 1]); the
 *      caller reads n_edges = row_ptr[n_atoms] (this needs the stream to
 *      finish) and sizes src and vec;
 *   2. etp_neighbor_fill, with the same pos, box and cutoff, writes src
 *      (DEVICE int32 [n_edges]) and vec (DEVICE float [n_edges][3]); vec also
 *      serves as scratch during the call.
 * ws: DEVICE workspace of at least etp_neighbor_workspace() bytes (contents
 * need not survive between the calls). Nothing is allocated, except that
 * ETP_FLAG_VALIDATE (the only flag of the fill) checks row_ptr before the
 * fill and, after it, that every row got exactly its count (positions that
 * changed between the calls fail it), synchronising the stream; without it
 * such rows hold -1 padding or are cut short, and their vec is NaN where the
 * source is -1. Errors: INVALID_ARGUMENT (negative n_atoms or n_edges, null
 * pointers, cutoff not positive and finite, box sides not positive and
 * finite, other flags), UNSUPPORTED (a box side below 2 * cutoff, n_edges >=
 * 2^31), WORKSPACE, INTERNAL (VALIDATE found a mismatch), HIP. The total
 * edge count must stay below 2^31 (row_ptr is int32). */
ETP_API etp_status etp_neighbor_workspace(int32_t n_atoms, const float *box, float cutoff, size_t *bytes);
ETP_API etp_status etp_neighbor_count(int32_t n_atoms, const float *pos, const float *box, float cutoff,
                                      int32_t *row_ptr, void *ws, size_t ws_bytes, void *stream);
ETP_API etp_status etp_neighbor_fill(int32_t n_atoms, const float *pos, const float *box, float cutoff,
                                     const int32_t *row_ptr, int64_t n_edges, int32_t *src, float *vec,
                                     uint32_t flags, void *ws, size_t ws_bytes, void *stream);

ETP_API const char *etp_status_string(etp_status s);

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
ETP_API int32_t etp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ETP_H */
