/*
 * etp_oracle.c -- float64 CPU oracle for the fused edge tensor-product
 * convolution (forward, VJP, VJP-of-VJP), its spherical harmonics, its
 * Clebsch-Gordan table and the stable CSR transpose.
 *
 * TEST INFRASTRUCTURE. This file is the checker, not the product. Only the
 * test suite, the package smoke check and the benchmark's CPU-baseline leg
 * may load the library built from it. It shares no source with the HIP
 * library and includes none of its headers.
 *
 * What it computes, and where that is stated:
 *  - The convolution is a Clebsch-Gordan (Wigner 3-j) tensor product of the
 *    source node's irrep features with the real spherical harmonics of the
 *    bond vector, scaled per edge/path/channel by a radial weight and summed
 *    into the destination node ("High-performance training and inference for
 *    deep equivariant interatomic potentials", review page, section "Proposed
 *    method": the tensor product with Wigner 3-j coefficients held in a
 *    compressed sparse form; "Machine Learning Interatomic Potentials:
 *    Advancing Open-Source Software...", section on the e3j backend: CG tensor
 *    products as the bottleneck of MACE/NequIP).
 *  - Forward, VJP and VJP-of-VJP are the three stages measured for the edge
 *    convolution ("How does FlashCart make equivariant interatomic potentials
 *    faster and more accurate?", section "Generated kernels beat SH baselines
 *    at high order"); forces are the VJP with respect to the bond vectors
 *    (same page, section on the SPICE-MACE-OFF model: energy and forces).
 *  - The pages give no formulas. The definitions below are textbook
 *    angular-momentum algebra under these readings:
 *      * SO(3) only, every triangle-allowed path (l1,l2,l3) kept, paths
 *        enumerated lexicographically with l3 <= l_max_out;
 *      * complex CG from Racah's closed form (Condon-Shortley phase);
 *      * real basis: m'>0 -> (Y^{-m'} + (-1)^{m'} Y^{m'})/sqrt2,
 *        m'<0 (k=|m'|) -> i(Y^{-k} - (-1)^k Y^{k})/sqrt2; the real coupling
 *        tensor is the real part of the transformed tensor when l1+l2+l3 is
 *        even and its imaginary part when odd;
 *      * real SH in "component" normalisation (sum_m Y_l^m^2 = 2l+1), order
 *        m = -l..l, z the polar axis, evaluated at r/|r|, derivatives with
 *        respect to the unnormalised r;
 *      * channel-wise ("uvu") paths: one weight per (edge, path, channel),
 *        one output block per path, no path normalisation;
 *      * layouts x[n][l*l + l + m][u], out[n][off_p + (m3+l3)][u] with
 *        off_p = sum_{q<p}(2 l3_q + 1), w[e][p][u], vec[e][3].
 *
 * Every floating-point quantity is double. Loops go edge by edge, path by
 * path, CG entry by CG entry, channel by channel, in that plain order. OpenMP
 * splits the outer loop over destination nodes (forward, dG) or over source
 * nodes (VJP and the VJP-of-VJP source terms), so that no two threads write
 * the same output.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_LMAX 4

/* ------------------------------------------------------------------------ */
/* Paths                                                                     */
/* ------------------------------------------------------------------------ */

/* Lexicographic (l1, l2, l3) with |l1-l2| <= l3 <= min(l1+l2, lout).
 * Writes up to cap triples into out (may be NULL) and returns the count. */
int oracle_paths(int lin, int lsh, int lout, int32_t *out, int cap)
{
    int n = 0;
    for (int l1 = 0; l1 <= lin; ++l1)
        for (int l2 = 0; l2 <= lsh; ++l2)
            for (int l3 = abs(l1 - l2); l3 <= l1 + l2 && l3 <= lout; ++l3) {
                if (out && n < cap) {
                    out[3 * n + 0] = l1;
                    out[3 * n + 1] = l2;
                    out[3 * n + 2] = l3;
                }
                ++n;
            }
    return n;
}

/* ------------------------------------------------------------------------ */
/* Clebsch-Gordan coefficients                                               */
/* ------------------------------------------------------------------------ */

static double factorial(int n)
{
    /* exact in double for n <= 18; the largest argument used is
     * l1 + l2 + l3 + 1 = 17 (l1, l2 <= 4, l3 <= 8) */
    double r = 1.0;
    for (int i = 2; i <= n; ++i)
        r *= i;
    return r;
}

/* <j1 m1 j2 m2 | J M>, Racah's closed form, Condon-Shortley phase. */
double oracle_cg_complex(int j1, int m1, int j2, int m2, int J, int M)
{
    if (M != m1 + m2)
        return 0.0;
    if (J < abs(j1 - j2) || J > j1 + j2)
        return 0.0;
    if (abs(m1) > j1 || abs(m2) > j2 || abs(M) > J)
        return 0.0;
    double pre = (2.0 * J + 1.0) * factorial(J + j1 - j2) * factorial(J - j1 + j2) *
                 factorial(j1 + j2 - J) / factorial(j1 + j2 + J + 1);
    pre *= factorial(J + M) * factorial(J - M) * factorial(j1 - m1) * factorial(j1 + m1) *
           factorial(j2 - m2) * factorial(j2 + m2);
    double s = 0.0;
    for (int k = 0; k <= j1 + j2 + J; ++k) {
        int d1 = j1 + j2 - J - k, d2 = j1 - m1 - k, d3 = j2 + m2 - k;
        int d4 = J - j2 + m1 + k, d5 = J - j1 - m2 + k;
        if (d1 < 0 || d2 < 0 || d3 < 0 || d4 < 0 || d5 < 0)
            continue;
        double den = factorial(k) * factorial(d1) * factorial(d2) * factorial(d3) *
                     factorial(d4) * factorial(d5);
        s += ((k & 1) ? -1.0 : 1.0) / den;
    }
    return sqrt(pre) * s;
}

/* Complex-to-real change of basis U_l, row = real index m', column = complex
 * m, both stored as m + l. */
static void real_basis(int l, double complex *U)
{
    int d = 2 * l + 1;
    const double h = 1.0 / sqrt(2.0);
    for (int i = 0; i < d * d; ++i)
        U[i] = 0.0;
    for (int mp = -l; mp <= l; ++mp) {
        int r = mp + l;
        if (mp > 0) {
            U[r * d + (-mp + l)] = h;
            U[r * d + (mp + l)] = ((mp & 1) ? -1.0 : 1.0) * h;
        } else if (mp == 0) {
            U[r * d + l] = 1.0;
        } else {
            int k = -mp;
            U[r * d + (mp + l)] = I * h;
            U[r * d + (k + l)] = -I * ((k & 1) ? -1.0 : 1.0) * h;
        }
    }
}

/* Dense real coupling tensor C[a][b][c] (a over 2l1+1, b over 2l2+1, c over
 * 2l3+1, indices m+l), l1, l2 <= 4 and l3 <= 8. Returns the largest magnitude of the discarded
 * (real or imaginary) part, so tests can check that it is round-off. */
double oracle_cg_real_dense(int l1, int l2, int l3, double *out)
{
    int d1 = 2 * l1 + 1, d2 = 2 * l2 + 1, d3 = 2 * l3 + 1;
    double complex U1[289], U2[289], U3[289]; /* up to l = 8 */
    real_basis(l1, U1);
    real_basis(l2, U2);
    real_basis(l3, U3);
    int odd = (l1 + l2 + l3) & 1;
    double discarded = 0.0;
    for (int a = 0; a < d1; ++a)
        for (int b = 0; b < d2; ++b)
            for (int c = 0; c < d3; ++c) {
                double complex s = 0.0;
                for (int al = 0; al < d1; ++al)
                    for (int be = 0; be < d2; ++be)
                        for (int ga = 0; ga < d3; ++ga) {
                            double cg = oracle_cg_complex(l1, al - l1, l2, be - l2, l3, ga - l3);
                            if (cg == 0.0)
                                continue;
                            s += U3[c * d3 + ga] * cg * conj(U1[a * d1 + al]) *
                                 conj(U2[b * d2 + be]);
                        }
                double keep = odd ? cimag(s) : creal(s);
                double drop = odd ? creal(s) : cimag(s);
                if (fabs(drop) > discarded)
                    discarded = fabs(drop);
                out[(a * d2 + b) * d3 + c] = keep;
            }
    return discarded;
}

/* Sparse table for all paths of (lin, lsh, lout): per path p the entries
 * ptr[p]..ptr[p+1]-1, each (m1, m2, m3) (signed m values) and a coefficient,
 * ordered by (m1, m2, m3) ascending, keeping |C| > 1e-12. Returns nnz; the
 * arrays may be NULL to query sizes (ptr needs P+1 slots). */
int oracle_cg_sparse(int lin, int lsh, int lout, int32_t *ptr, int8_t *m, double *val, int cap)
{
    int32_t paths[3 * 128];
    int P = oracle_paths(lin, lsh, lout, paths, 128);
    int nnz = 0;
    double dense[9 * 9 * 9];
    for (int p = 0; p < P; ++p) {
        int l1 = paths[3 * p], l2 = paths[3 * p + 1], l3 = paths[3 * p + 2];
        if (ptr)
            ptr[p] = nnz;
        oracle_cg_real_dense(l1, l2, l3, dense);
        for (int a = 0; a < 2 * l1 + 1; ++a)
            for (int b = 0; b < 2 * l2 + 1; ++b)
                for (int c = 0; c < 2 * l3 + 1; ++c) {
                    double v = dense[(a * (2 * l2 + 1) + b) * (2 * l3 + 1) + c];
                    if (fabs(v) <= 1e-12)
                        continue;
                    if (m && val && nnz < cap) {
                        m[3 * nnz + 0] = (int8_t)(a - l1);
                        m[3 * nnz + 1] = (int8_t)(b - l2);
                        m[3 * nnz + 2] = (int8_t)(c - l3);
                        val[nnz] = v;
                    }
                    ++nnz;
                }
    }
    if (ptr)
        ptr[P] = nnz;
    return nnz;
}

/* ------------------------------------------------------------------------ */
/* Real spherical harmonics with hyper-dual numbers                          */
/* ------------------------------------------------------------------------ */

/* a + b e1 + c e2 + d e1 e2 with e1^2 = e2^2 = 0: the e1 part carries one
 * first derivative, the e2 part another, the e1e2 part the mixed second. */
typedef struct {
    double a, b, c, d;
} hd;

static hd hd_const(double v) { hd r = {v, 0.0, 0.0, 0.0}; return r; }
static hd hd_add(hd x, hd y) { hd r = {x.a + y.a, x.b + y.b, x.c + y.c, x.d + y.d}; return r; }
static hd hd_sub(hd x, hd y) { hd r = {x.a - y.a, x.b - y.b, x.c - y.c, x.d - y.d}; return r; }
static hd hd_scale(hd x, double s) { hd r = {s * x.a, s * x.b, s * x.c, s * x.d}; return r; }
static hd hd_mul(hd x, hd y)
{
    hd r = {x.a * y.a, x.a * y.b + x.b * y.a, x.a * y.c + x.c * y.a,
            x.a * y.d + x.b * y.c + x.c * y.b + x.d * y.a};
    return r;
}
/* f(x) for a scalar function with derivatives f1 = f', f2 = f''. */
static hd hd_apply(hd x, double f, double f1, double f2)
{
    hd r = {f, f1 * x.b, f1 * x.c, f1 * x.d + f2 * x.b * x.c};
    return r;
}
static hd hd_rsqrt(hd x)
{
    double s = 1.0 / sqrt(x.a);
    return hd_apply(x, s, -0.5 * s / x.a, 0.75 * s / (x.a * x.a));
}

/* Y[l*l + l + m] for l <= L at n = r/|r| (component normalisation):
 *   Y_l^m = sqrt(2l+1) sqrt((l-|m|)!/(l+|m|)!) Q_l^|m|(n_z) * T_m,
 *   T_m = sqrt2 Re (n_x + i n_y)^m (m>0), 1 (m=0), sqrt2 Im (n_x+i n_y)^|m| (m<0),
 * with Q_l^m the associated Legendre function without the (1-z^2)^{m/2}
 * factor and without the Condon-Shortley phase:
 *   Q_m^m = (2m-1)!!, Q_{m+1}^m = (2m+1) z Q_m^m,
 *   Q_l^m = ((2l-1) z Q_{l-1}^m - (l+m-1) Q_{l-2}^m) / (l-m). */
static void sh_hd(int L, const hd r[3], hd *Y)
{
    hd r2 = hd_add(hd_add(hd_mul(r[0], r[0]), hd_mul(r[1], r[1])), hd_mul(r[2], r[2]));
    hd inv = hd_rsqrt(r2);
    hd nx = hd_mul(r[0], inv), ny = hd_mul(r[1], inv), nz = hd_mul(r[2], inv);

    hd Cm[OR_LMAX + 1], Sm[OR_LMAX + 1];
    Cm[0] = hd_const(1.0);
    Sm[0] = hd_const(0.0);
    for (int m = 0; m < L; ++m) {
        Cm[m + 1] = hd_sub(hd_mul(Cm[m], nx), hd_mul(Sm[m], ny));
        Sm[m + 1] = hd_add(hd_mul(Sm[m], nx), hd_mul(Cm[m], ny));
    }
    hd Q[OR_LMAX + 1][OR_LMAX + 1]; /* Q[l][m] */
    for (int m = 0; m <= L; ++m) {
        double dfact = 1.0;
        for (int k = 2 * m - 1; k > 1; k -= 2)
            dfact *= k;
        Q[m][m] = hd_const(dfact);
        if (m + 1 <= L)
            Q[m + 1][m] = hd_scale(hd_mul(nz, Q[m][m]), 2.0 * m + 1.0);
        for (int l = m + 2; l <= L; ++l)
            Q[l][m] = hd_scale(hd_sub(hd_scale(hd_mul(nz, Q[l - 1][m]), 2.0 * l - 1.0),
                                      hd_scale(Q[l - 2][m], l + m - 1.0)),
                               1.0 / (l - m));
    }
    for (int l = 0; l <= L; ++l)
        for (int m = -l; m <= l; ++m) {
            int am = abs(m);
            double norm = sqrt((2.0 * l + 1.0) * factorial(l - am) / factorial(l + am));
            hd t;
            if (m > 0)
                t = hd_scale(Cm[am], sqrt(2.0));
            else if (m == 0)
                t = hd_const(1.0);
            else
                t = hd_scale(Sm[am], sqrt(2.0));
            Y[l * l + l + m] = hd_scale(hd_mul(Q[l][am], t), norm);
        }
}

/* Y (D = (L+1)^2 values) at r; optionally dY[k][b] = dY_b/dr_k and, given a
 * direction v, HV[k][b] = d/dr_k (grad Y_b . v). Any of dY, v, HV may be
 * NULL (HV needs v). */
void oracle_sh_point(int L, const double r[3], const double *v, double *Y, double *dY, double *HV)
{
    int D = (L + 1) * (L + 1);
    hd rr[3], out[(OR_LMAX + 1) * (OR_LMAX + 1)];
    if (!dY && !HV) {
        for (int i = 0; i < 3; ++i)
            rr[i] = hd_const(r[i]);
        sh_hd(L, rr, out);
        for (int b = 0; b < D; ++b)
            Y[b] = out[b].a;
        return;
    }
    for (int k = 0; k < 3; ++k) {
        for (int i = 0; i < 3; ++i) {
            rr[i].a = r[i];
            rr[i].b = (i == k) ? 1.0 : 0.0;
            rr[i].c = v ? v[i] : 0.0;
            rr[i].d = 0.0;
        }
        sh_hd(L, rr, out);
        for (int b = 0; b < D; ++b) {
            if (k == 0 && Y)
                Y[b] = out[b].a;
            if (dY)
                dY[k * D + b] = out[b].b;
            if (HV)
                HV[k * D + b] = out[b].d;
        }
    }
}

/* Batched SH over edges: Y[e][D], dY[e][3][D] (nullable). */
void oracle_sh(int L, int64_t n, const double *vec, double *Y, double *dY)
{
    int D = (L + 1) * (L + 1);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e)
        oracle_sh_point(L, vec + 3 * e, NULL, Y + e * D, dY ? dY + e * 3 * D : NULL, NULL);
}

/* ------------------------------------------------------------------------ */
/* Stable CSR transpose                                                      */
/* ------------------------------------------------------------------------ */

/* Counting sort of edge ids by source, ties kept in edge-id order.
 * src_ptr[n_src+1], perm[E] (edge ids), perm_dst[E] (destination of perm[k]). */
void oracle_transpose(int n_dst, int n_src, const int32_t *row_ptr, const int32_t *src,
                      int32_t *src_ptr, int32_t *perm, int32_t *perm_dst)
{
    int64_t E = row_ptr[n_dst];
    int64_t *cursor = (int64_t *)calloc((size_t)n_src + 1, sizeof(int64_t));
    for (int j = 0; j <= n_src; ++j)
        src_ptr[j] = 0;
    for (int64_t e = 0; e < E; ++e)
        src_ptr[src[e] + 1] += 1;
    for (int j = 0; j < n_src; ++j)
        src_ptr[j + 1] += src_ptr[j];
    for (int j = 0; j < n_src; ++j)
        cursor[j] = src_ptr[j];
    for (int i = 0; i < n_dst; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            int64_t k = cursor[src[e]]++;
            perm[k] = (int32_t)e;
            perm_dst[k] = i;
        }
    free(cursor);
}

/* ------------------------------------------------------------------------ */
/* The convolution                                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
    int P, nnz, Din, Dsh, Dout; /* Din, Dout per channel */
    int32_t path[3 * 128];
    int32_t off[129];           /* output block offset per path (per channel) */
    int32_t ptr[129];
    int8_t *m;
    double *val;
} table;

static int table_make(int lin, int lsh, int lout, table *t)
{
    if (lin < 0 || lsh < 0 || lout < 0 || lin > OR_LMAX || lsh > OR_LMAX || lout > OR_LMAX)
        return -1;
    t->P = oracle_paths(lin, lsh, lout, t->path, 128);
    t->nnz = oracle_cg_sparse(lin, lsh, lout, NULL, NULL, NULL, 0);
    t->m = (int8_t *)malloc((size_t)3 * t->nnz);
    t->val = (double *)malloc(sizeof(double) * t->nnz);
    oracle_cg_sparse(lin, lsh, lout, t->ptr, t->m, t->val, t->nnz);
    t->Din = (lin + 1) * (lin + 1);
    t->Dsh = (lsh + 1) * (lsh + 1);
    int off = 0;
    for (int p = 0; p < t->P; ++p) {
        t->off[p] = off;
        off += 2 * t->path[3 * p + 2] + 1;
    }
    t->off[t->P] = off;
    t->Dout = off;
    return 0;
}

static void table_free(table *t)
{
    free(t->m);
    free(t->val);
}

/* One CG entry t of path p, resolved to row indices (per channel):
 * a = x row, b = Y index, c = out row. */
typedef struct {
    int a, b, c;
    double C;
} entry;

static entry entry_of(const table *t, int p, int k)
{
    int l1 = t->path[3 * p], l2 = t->path[3 * p + 1], l3 = t->path[3 * p + 2];
    entry en;
    en.a = l1 * l1 + l1 + t->m[3 * k + 0];
    en.b = l2 * l2 + l2 + t->m[3 * k + 1];
    en.c = t->off[p] + l3 + t->m[3 * k + 2];
    en.C = t->val[k];
    return en;
}

int oracle_dims(int lin, int lsh, int lout, int32_t *dims /* P, nnz, Din, Dsh, Dout */)
{
    table t;
    if (table_make(lin, lsh, lout, &t))
        return -1;
    dims[0] = t.P;
    dims[1] = t.nnz;
    dims[2] = t.Din;
    dims[3] = t.Dsh;
    dims[4] = t.Dout;
    table_free(&t);
    return 0;
}

/* out[i][c][u] = sum_{e in in(i)} sum_p w[e][p][u] sum_{t in p} C_t Y_b(vec_e) x[src_e][a][u] */
int oracle_fwd(int lin, int lsh, int lout, int C, int n_dst, const int32_t *row_ptr,
               const int32_t *src, const double *vec, const double *x, const double *w,
               double *out)
{
    table t;
    if (table_make(lin, lsh, lout, &t))
        return -1;
    const int P = t.P, Din = t.Din, Dout = t.Dout, L2 = lsh;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n_dst; ++i) {
        double Y[25];
        double *oi = out + (int64_t)i * Dout * C;
        for (int q = 0; q < Dout * C; ++q)
            oi[q] = 0.0;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            const double *xj = x + (int64_t)src[e] * Din * C;
            const double *we = w + e * P * C;
            oracle_sh_point(L2, vec + 3 * e, NULL, Y, NULL, NULL);
            for (int p = 0; p < P; ++p)
                for (int k = t.ptr[p]; k < t.ptr[p + 1]; ++k) {
                    entry en = entry_of(&t, p, k);
                    for (int u = 0; u < C; ++u)
                        oi[en.c * C + u] += we[p * C + u] * en.C * Y[en.b] * xj[en.a * C + u];
                }
        }
    }
    table_free(&t);
    return 0;
}

/* VJP of the forward given G = dL/dout:
 *   gx[j][a][u] = sum_{e in out(j)} sum_p w[e][p][u] sum_{t: a_t=a} C_t Y_b G[i][c][u]
 *   gw[e][p][u] = sum_t C_t Y_b x[j][a][u] G[i][c][u]
 *   gr[e][k]    = sum_b dY_b/dr_k * Z_b,  Z_b = sum_{p,u} w sum_{t: b_t=b} C_t x G
 * Any output may be NULL. The source-segmented sum uses this file's own
 * transpose so that threads own disjoint gx rows. */
int oracle_vjp(int lin, int lsh, int lout, int C, int n_dst, int n_src, const int32_t *row_ptr,
               const int32_t *src, const double *vec, const double *x, const double *w,
               const double *G, double *gx, double *gw, double *gr)
{
    table t;
    if (table_make(lin, lsh, lout, &t))
        return -1;
    const int P = t.P, Din = t.Din, Dsh = t.Dsh, Dout = t.Dout, L2 = lsh;
    int64_t E = row_ptr[n_dst];
    int32_t *sp = (int32_t *)malloc(sizeof(int32_t) * ((size_t)n_src + 1));
    int32_t *perm = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    int32_t *pdst = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    oracle_transpose(n_dst, n_src, row_ptr, src, sp, perm, pdst);
#pragma omp parallel for schedule(static)
    for (int j = 0; j < n_src; ++j) {
        double Y[25], dY[75], Z[25];
        const double *xj = x + (int64_t)j * Din * C;
        double *gxj = gx ? gx + (int64_t)j * Din * C : NULL;
        if (gxj)
            for (int q = 0; q < Din * C; ++q)
                gxj[q] = 0.0;
        for (int64_t k = sp[j]; k < sp[j + 1]; ++k) {
            int64_t e = perm[k];
            int i = pdst[k];
            const double *we = w + e * P * C;
            const double *Gi = G + (int64_t)i * Dout * C;
            oracle_sh_point(L2, vec + 3 * e, NULL, Y, dY, NULL);
            for (int b = 0; b < Dsh; ++b)
                Z[b] = 0.0;
            if (gw)
                for (int q = 0; q < P * C; ++q)
                    gw[e * P * C + q] = 0.0;
            for (int p = 0; p < P; ++p)
                for (int kk = t.ptr[p]; kk < t.ptr[p + 1]; ++kk) {
                    entry en = entry_of(&t, p, kk);
                    for (int u = 0; u < C; ++u) {
                        double g = Gi[en.c * C + u];
                        double xa = xj[en.a * C + u];
                        double wv = we[p * C + u];
                        if (gxj)
                            gxj[en.a * C + u] += wv * en.C * Y[en.b] * g;
                        if (gw)
                            gw[e * P * C + p * C + u] += en.C * Y[en.b] * xa * g;
                        Z[en.b] += en.C * wv * xa * g;
                    }
                }
            if (gr)
                for (int kd = 0; kd < 3; ++kd) {
                    double s = 0.0;
                    for (int b = 0; b < Dsh; ++b)
                        s += dY[kd * Dsh + b] * Z[b];
                    gr[e * 3 + kd] = s;
                }
        }
    }
    free(sp);
    free(perm);
    free(pdst);
    table_free(&t);
    return 0;
}

/* VJP of the VJP. With cotangents X' (like x), W' (like w), R' (like vec) on
 * (gx, gw, gr), and Yd_b = grad Y_b . R'_e, H_b = d/dr (grad Y_b . R'_e):
 *   dG[i][c][u] = sum_{e in in(i)} sum_{t: c_t=c} C_t [Y_b (w X'_a + W' x_a) + Yd_b w x_a]
 *   dx[j][a][u] = sum_{e in out(j)} sum_{p,t: a_t=a} C_t G_c [Y_b W' + Yd_b w]
 *   dw[e][p][u] = sum_t C_t G_c [Y_b X'_a + Yd_b x_a]
 *   dr[e]       = sum_b Z1_b grad Y_b + Z2_b H_b,
 *       Z1_b = sum_{p,u} sum_{t: b} C_t G_c (w X'_a + W' x_a),
 *       Z2_b = sum_{p,u} sum_{t: b} C_t G_c w x_a.
 * X', W', R' may be NULL (zero). Outputs may be NULL (not computed). */
int oracle_vjp2(int lin, int lsh, int lout, int C, int n_dst, int n_src, const int32_t *row_ptr,
                const int32_t *src, const double *vec, const double *x, const double *w,
                const double *G, const double *Xp, const double *Wp, const double *Rp,
                double *dx, double *dw, double *dr, double *dG)
{
    table t;
    if (table_make(lin, lsh, lout, &t))
        return -1;
    const int P = t.P, Din = t.Din, Dsh = t.Dsh, Dout = t.Dout, L2 = lsh;
    int64_t E = row_ptr[n_dst];
    static const double zero3[3] = {0.0, 0.0, 0.0};

    /* destination pass: dG */
    if (dG) {
#pragma omp parallel for schedule(static)
        for (int i = 0; i < n_dst; ++i) {
            double Y[25], dY[75];
            double *oi = dG + (int64_t)i * Dout * C;
            for (int q = 0; q < Dout * C; ++q)
                oi[q] = 0.0;
            for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
                int j = src[e];
                const double *xj = x + (int64_t)j * Din * C;
                const double *Xj = Xp ? Xp + (int64_t)j * Din * C : NULL;
                const double *we = w + e * P * C;
                const double *We = Wp ? Wp + e * P * C : NULL;
                const double *rp = Rp ? Rp + 3 * e : zero3;
                oracle_sh_point(L2, vec + 3 * e, NULL, Y, dY, NULL);
                double Yd[25];
                for (int b = 0; b < Dsh; ++b)
                    Yd[b] = dY[b] * rp[0] + dY[Dsh + b] * rp[1] + dY[2 * Dsh + b] * rp[2];
                for (int p = 0; p < P; ++p)
                    for (int k = t.ptr[p]; k < t.ptr[p + 1]; ++k) {
                        entry en = entry_of(&t, p, k);
                        for (int u = 0; u < C; ++u) {
                            double wv = we[p * C + u];
                            double xa = xj[en.a * C + u];
                            double Xa = Xj ? Xj[en.a * C + u] : 0.0;
                            double Wv = We ? We[p * C + u] : 0.0;
                            oi[en.c * C + u] +=
                                en.C * (Y[en.b] * (wv * Xa + Wv * xa) + Yd[en.b] * wv * xa);
                        }
                    }
            }
        }
    }

    /* source pass: dx, dw, dr */
    if (dx || dw || dr) {
        int32_t *sp = (int32_t *)malloc(sizeof(int32_t) * ((size_t)n_src + 1));
        int32_t *perm = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
        int32_t *pdst = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
        oracle_transpose(n_dst, n_src, row_ptr, src, sp, perm, pdst);
#pragma omp parallel for schedule(static)
        for (int j = 0; j < n_src; ++j) {
            double Y[25], dY[75], HV[75], Yd[25], Z1[25], Z2[25];
            const double *xj = x + (int64_t)j * Din * C;
            const double *Xj = Xp ? Xp + (int64_t)j * Din * C : NULL;
            double *dxj = dx ? dx + (int64_t)j * Din * C : NULL;
            if (dxj)
                for (int q = 0; q < Din * C; ++q)
                    dxj[q] = 0.0;
            for (int64_t k = sp[j]; k < sp[j + 1]; ++k) {
                int64_t e = perm[k];
                int i = pdst[k];
                const double *we = w + e * P * C;
                const double *We = Wp ? Wp + e * P * C : NULL;
                const double *Gi = G + (int64_t)i * Dout * C;
                const double *rp = Rp ? Rp + 3 * e : zero3;
                oracle_sh_point(L2, vec + 3 * e, rp, Y, dY, HV);
                for (int b = 0; b < Dsh; ++b) {
                    Yd[b] = dY[b] * rp[0] + dY[Dsh + b] * rp[1] + dY[2 * Dsh + b] * rp[2];
                    Z1[b] = 0.0;
                    Z2[b] = 0.0;
                }
                if (dw)
                    for (int q = 0; q < P * C; ++q)
                        dw[e * P * C + q] = 0.0;
                for (int p = 0; p < P; ++p)
                    for (int kk = t.ptr[p]; kk < t.ptr[p + 1]; ++kk) {
                        entry en = entry_of(&t, p, kk);
                        for (int u = 0; u < C; ++u) {
                            double g = Gi[en.c * C + u];
                            double wv = we[p * C + u];
                            double xa = xj[en.a * C + u];
                            double Xa = Xj ? Xj[en.a * C + u] : 0.0;
                            double Wv = We ? We[p * C + u] : 0.0;
                            if (dxj)
                                dxj[en.a * C + u] += en.C * g * (Y[en.b] * Wv + Yd[en.b] * wv);
                            if (dw)
                                dw[e * P * C + p * C + u] += en.C * g * (Y[en.b] * Xa + Yd[en.b] * xa);
                            Z1[en.b] += en.C * g * (wv * Xa + Wv * xa);
                            Z2[en.b] += en.C * g * wv * xa;
                        }
                    }
                if (dr)
                    for (int kd = 0; kd < 3; ++kd) {
                        double s = 0.0;
                        for (int b = 0; b < Dsh; ++b)
                            s += Z1[b] * dY[kd * Dsh + b] + Z2[b] * HV[kd * Dsh + b];
                        dr[e * 3 + kd] = s;
                    }
            }
        }
        free(sp);
        free(perm);
        free(pdst);
    }
    table_free(&t);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Channel mixing after the convolution                                      */
/* ------------------------------------------------------------------------ */

/* A per-irrep linear layer on the convolution output: for every output
 * order l, the channels of all paths with l3 = l (in path order) are mixed
 * by one dense matrix W_l of (n_l * C) rows and C columns, the same for every
 * component m (so the map commutes with rotations):
 *   y[i][l*l + l + m][v] = sum_{p: l3_p = l} sum_u W_l[(q_p*C + u)*C + v] * out[i][off_p + l + m][u]
 * with q_p the rank of p among the paths of order l. W holds W_0, W_1, ...,
 * W_lout back to back. The pages name the dense channel contraction that
 * follows the tensor product ("Scaling the leading accuracy of deep
 * equivariant models to biomolecular simulations of realistic size",
 * section "Proposed method") but not its form; this is the plainest
 * equivariant reading (one matrix per output order, shared by its
 * components). */
int oracle_channel_mix(int lin, int lsh, int lout, int C, int n, const double *out, const double *W, double *y)
{
    table t;
    if (table_make(lin, lsh, lout, &t))
        return -1;
    const int Dout = t.Dout, Dy = (lout + 1) * (lout + 1);
    /* start of W_l and the rank of every path among those of its order */
    int64_t wofs[OR_LMAX + 2];
    int rank[128], count[OR_LMAX + 1] = {0};
    for (int p = 0; p < t.P; ++p) {
        const int l3 = t.path[3 * p + 2];
        rank[p] = count[l3]++;
    }
    wofs[0] = 0;
    for (int l = 0; l <= lout; ++l)
        wofs[l + 1] = wofs[l] + (int64_t)count[l] * C * C;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n; ++i) {
        double *yi = y + (int64_t)i * Dy * C;
        for (int q = 0; q < Dy * C; ++q)
            yi[q] = 0.0;
        for (int p = 0; p < t.P; ++p) {
            const int l = t.path[3 * p + 2];
            const double *Wl = W + wofs[l] + (int64_t)rank[p] * C * C;
            for (int mi = 0; mi < 2 * l + 1; ++mi) {
                const double *o = out + ((int64_t)i * Dout + t.off[p] + mi) * C;
                double *yr = yi + (int64_t)(l * l + mi) * C;
                for (int u = 0; u < C; ++u)
                    for (int v = 0; v < C; ++v)
                        yr[v] += Wl[(int64_t)u * C + v] * o[u];
            }
        }
    }
    table_free(&t);
    return 0;
}

/* VJP of the channel mixing with respect to its input (the mixing is linear,
 * so this is the transposed map): gin[i][off_p + m][u] = sum_v W_l[(q_p C + u)
 * C + v] gy[i][l*l + m][v] for every path p of order l = l3_p. */
int oracle_channel_mix_vjp(int lin, int lsh, int lout, int C, int n, const double *gy, const double *W, double *gin)
{
    table t;
    if (table_make(lin, lsh, lout, &t))
        return -1;
    const int Dout = t.Dout, Dy = (lout + 1) * (lout + 1);
    int64_t wofs[OR_LMAX + 2];
    int prank[128], pcount[OR_LMAX + 1] = {0};
    for (int p = 0; p < t.P; ++p) {
        const int l3 = t.path[3 * p + 2];
        prank[p] = pcount[l3]++;
    }
    wofs[0] = 0;
    for (int l = 0; l <= lout; ++l)
        wofs[l + 1] = wofs[l] + (int64_t)pcount[l] * C * C;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n; ++i) {
        for (int p = 0; p < t.P; ++p) {
            const int l = t.path[3 * p + 2];
            const double *Wl = W + wofs[l] + (int64_t)prank[p] * C * C;
            for (int mi = 0; mi < 2 * l + 1; ++mi) {
                const double *gr = gy + ((int64_t)i * Dy + l * l + mi) * C;
                double *o = gin + ((int64_t)i * Dout + t.off[p] + mi) * C;
                for (int u = 0; u < C; ++u) {
                    double acc = 0.0;
                    for (int v = 0; v < C; ++v)
                        acc += Wl[(int64_t)u * C + v] * gr[v];
                    o[u] = acc;
                }
            }
        }
    }
    table_free(&t);
    return 0;
}

/* Gradient of the channel mixing with respect to its weights (the mixing is
 * linear in W; a sum over every node and component):
 * gW_l[(q_p C + u) C + v] = sum_i sum_m out[i][off_p + m][u] gy[i][l*l + m][v]
 * for every path p of order l = l3_p. Nodes in index order, serially. */
int oracle_channel_mix_wgrad(int lin, int lsh, int lout, int C, int n, const double *out, const double *gy, double *gW)
{
    table t;
    if (table_make(lin, lsh, lout, &t))
        return -1;
    const int Dout = t.Dout, Dy = (lout + 1) * (lout + 1);
    int64_t wofs[OR_LMAX + 2];
    int prank[128], pcount[OR_LMAX + 1] = {0};
    for (int p = 0; p < t.P; ++p) {
        const int l3 = t.path[3 * p + 2];
        prank[p] = pcount[l3]++;
    }
    wofs[0] = 0;
    for (int l = 0; l <= lout; ++l)
        wofs[l + 1] = wofs[l] + (int64_t)pcount[l] * C * C;
    for (int64_t q = 0; q < wofs[lout + 1]; ++q)
        gW[q] = 0.0;
#pragma omp parallel for schedule(static)
    for (int p = 0; p < t.P; ++p) {  /* each path owns its block of gW */
        const int l = t.path[3 * p + 2];
        double *G = gW + wofs[l] + (int64_t)prank[p] * C * C;
        for (int i = 0; i < n; ++i)
            for (int mi = 0; mi < 2 * l + 1; ++mi) {
                const double *o = out + ((int64_t)i * Dout + t.off[p] + mi) * C;
                const double *gyr = gy + ((int64_t)i * Dy + l * l + mi) * C;
                for (int u = 0; u < C; ++u)
                    for (int v = 0; v < C; ++v)
                        G[(int64_t)u * C + v] += o[u] * gyr[v];
            }
    }
    table_free(&t);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Forces on the atoms                                                       */
/* ------------------------------------------------------------------------ */

/* With vec_e = pos[src_e] - pos[dst_e] (from the receiving atom to its
 * neighbour) and gr_e = dE/dvec_e, the chain rule gives
 * dE/dpos[k] = sum_{e: src_e = k} gr_e - sum_{e: dst_e = k} gr_e, and the
 * force F = -dE/dpos (energy and forces from one model: "How does FlashCart
 * make equivariant interatomic potentials faster and more accurate?",
 * section on the SPICE-MACE-OFF model). F has max(n_dst, n_src) rows; edge
 * by edge, in edge order. */
void oracle_edge_forces(int n_dst, int n_src, const int32_t *row_ptr, const int32_t *src, const double *gr,
                        double *F)
{
    const int n = n_dst > n_src ? n_dst : n_src;
    for (int k = 0; k < 3 * n; ++k)
        F[k] = 0.0;
    for (int i = 0; i < n_dst; ++i)
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e)
            for (int c = 0; c < 3; ++c) {
                F[3 * i + c] += gr[3 * e + c];
                F[3 * (int64_t)src[e] + c] -= gr[3 * e + c];
            }
}

/* ------------------------------------------------------------------------ */
/* Node-local correlation product                                            */
/* ------------------------------------------------------------------------ */

/* The node-local product ladder of "How does FlashCart make equivariant
 * interatomic potentials faster and more accurate?" (section "Generated
 * kernels beat SH baselines at high order"): weighted products applied step
 * by step, each result truncated to orders <= L. The page gives no formula;
 * the reading here, channel by channel (channel u only meets channel u):
 *   B_1 = A
 *   B_{k+1}[l3, m3, u] = sum over paths p = (l1, l2, l3) of W[k-1][p][u]
 *                        sum_{(m1, m2, m3)} C_p[m1, m2, m3] B_k[l1, m1, u] A[l2, m2, u]
 *   out = B_1 + B_2 + ... + B_nu
 * with the convolution's path list and real CG (l1, l2, l3 <= L). A and out
 * have the node-feature layout [n][(L+1)^2][C]; W is [nu-1][P][C]. */
int oracle_node_product(int L, int C, int n, int nu, const double *A, const double *W, double *out)
{
    table t;
    if (nu < 1 || table_make(L, L, L, &t))
        return -1;
    const int D = (L + 1) * (L + 1), P = t.P;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n; ++i) {
        double *B = (double *)malloc(sizeof(double) * D * C);
        double *NB = (double *)malloc(sizeof(double) * D * C);
        const double *Ai = A + (int64_t)i * D * C;
        double *oi = out + (int64_t)i * D * C;
        for (int q = 0; q < D * C; ++q) {
            B[q] = Ai[q];
            oi[q] = Ai[q];
        }
        for (int k = 1; k < nu; ++k) {
            for (int q = 0; q < D * C; ++q)
                NB[q] = 0.0;
            for (int p = 0; p < P; ++p) {
                const int l1 = t.path[3 * p], l2 = t.path[3 * p + 1], l3 = t.path[3 * p + 2];
                const double *Wp = W + ((int64_t)(k - 1) * P + p) * C;
                for (int q = t.ptr[p]; q < t.ptr[p + 1]; ++q) {
                    const int r1 = l1 * l1 + l1 + t.m[3 * q], r2 = l2 * l2 + l2 + t.m[3 * q + 1];
                    const int r3 = l3 * l3 + l3 + t.m[3 * q + 2];
                    for (int u = 0; u < C; ++u)
                        NB[r3 * C + u] += Wp[u] * t.val[q] * B[r1 * C + u] * Ai[r2 * C + u];
                }
            }
            for (int q = 0; q < D * C; ++q) {
                B[q] = NB[q];
                oi[q] += NB[q];
            }
        }
        free(B);
        free(NB);
    }
    table_free(&t);
    return 0;
}

/* VJP of the node-local product with respect to A (what forces need: A is
 * built from the positions): gA = d<G, out>/dA by reverse mode over the
 * ladder, every B_k kept. With Bbar_nu = G:
 *   Bbar_k = G + sum_p W[k-1][p] sum C A[l2,m2] Bbar_{k+1}[l3,m3]   (into [l1,m1])
 *   gA    += sum_p W[k-1][p] sum C B_k[l1,m1] Bbar_{k+1}[l3,m3]     (into [l2,m2])
 * for k = nu-1 .. 1, then gA += Bbar_1 (B_1 = A). */
int oracle_node_product_vjp(int L, int C, int n, int nu, const double *A, const double *W, const double *G,
                            double *gA)
{
    table t;
    if (nu < 1 || table_make(L, L, L, &t))
        return -1;
    const int D = (L + 1) * (L + 1), P = t.P;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n; ++i) {
        const double *Ai = A + (int64_t)i * D * C, *Gi = G + (int64_t)i * D * C;
        double *gi = gA + (int64_t)i * D * C;
        double *B = (double *)malloc(sizeof(double) * (size_t)nu * D * C); /* B_1 .. B_nu */
        double *bb = (double *)malloc(sizeof(double) * D * C);
        double *nbb = (double *)malloc(sizeof(double) * D * C);
        for (int q = 0; q < D * C; ++q)
            B[q] = Ai[q];
        for (int k = 1; k < nu; ++k) {
            double *Bk = B + (int64_t)(k - 1) * D * C, *Bn = B + (int64_t)k * D * C;
            for (int q = 0; q < D * C; ++q)
                Bn[q] = 0.0;
            for (int p = 0; p < P; ++p) {
                const int l1 = t.path[3 * p], l2 = t.path[3 * p + 1], l3 = t.path[3 * p + 2];
                const double *Wv = W + ((int64_t)(k - 1) * P + p) * C;
                for (int q = t.ptr[p]; q < t.ptr[p + 1]; ++q) {
                    const int s1 = l1 * l1 + l1 + t.m[3 * q], s2 = l2 * l2 + l2 + t.m[3 * q + 1];
                    const int s3 = l3 * l3 + l3 + t.m[3 * q + 2];
                    for (int u = 0; u < C; ++u)
                        Bn[s3 * C + u] += Wv[u] * t.val[q] * Bk[s1 * C + u] * Ai[s2 * C + u];
                }
            }
        }
        for (int q = 0; q < D * C; ++q) {
            bb[q] = Gi[q];
            gi[q] = 0.0;
        }
        for (int k = nu - 1; k >= 1; --k) {
            const double *Bk = B + (int64_t)(k - 1) * D * C;
            for (int q = 0; q < D * C; ++q)
                nbb[q] = Gi[q];
            for (int p = 0; p < P; ++p) {
                const int l1 = t.path[3 * p], l2 = t.path[3 * p + 1], l3 = t.path[3 * p + 2];
                const double *Wv = W + ((int64_t)(k - 1) * P + p) * C;
                for (int q = t.ptr[p]; q < t.ptr[p + 1]; ++q) {
                    const int s1 = l1 * l1 + l1 + t.m[3 * q], s2 = l2 * l2 + l2 + t.m[3 * q + 1];
                    const int s3 = l3 * l3 + l3 + t.m[3 * q + 2];
                    for (int u = 0; u < C; ++u) {
                        const double s = Wv[u] * t.val[q] * bb[s3 * C + u];
                        nbb[s1 * C + u] += s * Ai[s2 * C + u];
                        gi[s2 * C + u] += s * Bk[s1 * C + u];
                    }
                }
            }
            for (int q = 0; q < D * C; ++q)
                bb[q] = nbb[q];
        }
        for (int q = 0; q < D * C; ++q)
            gi[q] += bb[q];
        free(B);
        free(bb);
        free(nbb);
    }
    table_free(&t);
    return 0;
}

/* Gradient of <G, out> of the node-local product with respect to its weights
 * (a sum over every node; training the ladder): with Bbar_{k+1} the adjoint of
 * B_{k+1} from the reverse recursion of oracle_node_product_vjp,
 *   gW[k-1][p][u] = sum_i sum_{(m1, m2, m3) in p} C * Bbar_{k+1}[l3,m3,u] * B_k[l1,m1,u] * A[l2,m2,u]
 * for k = 1 .. nu-1. Nodes in index order, serially. */
int oracle_node_product_wgrad(int L, int C, int n, int nu, const double *A, const double *W, const double *G,
                              double *gW)
{
    table t;
    if (nu < 1 || table_make(L, L, L, &t))
        return -1;
    const int D = (L + 1) * (L + 1), P = t.P;
    for (int64_t q = 0; q < (int64_t)(nu - 1) * P * C; ++q)
        gW[q] = 0.0;
    double *B = (double *)malloc(sizeof(double) * (size_t)nu * D * C); /* B_1 .. B_nu of one node */
    double *adj = (double *)malloc(sizeof(double) * D * C);            /* adjoint of B_{k+1} */
    double *nadj = (double *)malloc(sizeof(double) * D * C);
    for (int i = 0; i < n; ++i) {
        const double *Ai = A + (int64_t)i * D * C, *Gi = G + (int64_t)i * D * C;
        for (int q = 0; q < D * C; ++q)
            B[q] = Ai[q];
        for (int k = 1; k < nu; ++k) {
            double *Bk = B + (int64_t)(k - 1) * D * C, *Bn = B + (int64_t)k * D * C;
            for (int q = 0; q < D * C; ++q)
                Bn[q] = 0.0;
            for (int p = 0; p < P; ++p) {
                const int l1 = t.path[3 * p], l2 = t.path[3 * p + 1], l3 = t.path[3 * p + 2];
                const double *Wv = W + ((int64_t)(k - 1) * P + p) * C;
                for (int q = t.ptr[p]; q < t.ptr[p + 1]; ++q) {
                    const int s1 = l1 * l1 + l1 + t.m[3 * q], s2 = l2 * l2 + l2 + t.m[3 * q + 1];
                    const int s3 = l3 * l3 + l3 + t.m[3 * q + 2];
                    for (int u = 0; u < C; ++u)
                        Bn[s3 * C + u] += Wv[u] * t.val[q] * Bk[s1 * C + u] * Ai[s2 * C + u];
                }
            }
        }
        for (int q = 0; q < D * C; ++q)
            adj[q] = Gi[q];                       /* adjoint of B_nu */
        for (int k = nu - 1; k >= 1; --k) {      /* step k maps B_k to B_{k+1} */
            const double *Bk = B + (int64_t)(k - 1) * D * C;
            for (int q = 0; q < D * C; ++q)
                nadj[q] = Gi[q];
            for (int p = 0; p < P; ++p) {
                const int l1 = t.path[3 * p], l2 = t.path[3 * p + 1], l3 = t.path[3 * p + 2];
                const double *Wv = W + ((int64_t)(k - 1) * P + p) * C;
                double *gWp = gW + ((int64_t)(k - 1) * P + p) * C;
                for (int q = t.ptr[p]; q < t.ptr[p + 1]; ++q) {
                    const int s1 = l1 * l1 + l1 + t.m[3 * q], s2 = l2 * l2 + l2 + t.m[3 * q + 1];
                    const int s3 = l3 * l3 + l3 + t.m[3 * q + 2];
                    for (int u = 0; u < C; ++u) {
                        gWp[u] += t.val[q] * adj[s3 * C + u] * Bk[s1 * C + u] * Ai[s2 * C + u];
                        nadj[s1 * C + u] += Wv[u] * t.val[q] * adj[s3 * C + u] * Ai[s2 * C + u];
                    }
                }
            }
            for (int q = 0; q < D * C; ++q)
                adj[q] = nadj[q];
        }
    }
    free(B);
    free(adj);
    free(nadj);
    table_free(&t);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Neighbour list                                                            */
/* ------------------------------------------------------------------------ */

/* Periodic neighbour list of n atoms in an orthorhombic box (each side at
 * least twice the cutoff): edge (i <- j) for every j != i whose minimum-image
 * distance is strictly below rc, rows sorted by j; vec = the minimum-image
 * displacement pos[j] - pos[i] (the graph the convolution walks: "edges per
 * atom" in "How does FlashCart make equivariant interatomic potentials faster
 * and more accurate?", section on the SPICE-MACE-OFF model). The cutoff test
 * decides an integer from floating point, so it is taken in float32 with the
 * operations spelled out (wrap q = p - L floor(p / L), d = q_j - q_i,
 * d -= L rint(d / L), r2 = dx dx + dy dy + dz dz as fused multiply-adds),
 * which any implementation of this contract reproduces bit for bit. Brute
 * force over all pairs. Returns the number of edges; src / vec are written
 * only when not NULL (then they must hold that many). */
static float or_wrap(float p, float L) { return fmaf(-L, floorf(p / L), p); }

/* Row i of the list: writes (when not NULL) its sources, ascending, and
 * their vectors; returns the row length. */
int oracle_neighbor_row(int n, const float *pos, const float *box, float rc, int i, int32_t *src, float *vec)
{
    const float rc2 = rc * rc;
    float qi[3];
    int k = 0;
    for (int c = 0; c < 3; ++c)
        qi[c] = or_wrap(pos[3 * i + c], box[c]);
    for (int j = 0; j < n; ++j) {
        if (j == i)
            continue;
        float d[3];
        for (int c = 0; c < 3; ++c) {
            const float dc = or_wrap(pos[3 * j + c], box[c]) - qi[c];
            d[c] = fmaf(-box[c], rintf(dc / box[c]), dc);
        }
        const float r2 = fmaf(d[2], d[2], fmaf(d[1], d[1], d[0] * d[0]));
        if (r2 < rc2) {
            if (src)
                src[k] = j;
            if (vec)
                for (int c = 0; c < 3; ++c)
                    vec[3 * k + c] = d[c];
            ++k;
        }
    }
    return k;
}

int64_t oracle_neighbors(int n, const float *pos, const float *box, float rc, int32_t *row_ptr, int32_t *src,
                         float *vec)
{
    int64_t e = 0;
    if (row_ptr)
        row_ptr[0] = 0;
    for (int i = 0; i < n; ++i) {
        e += oracle_neighbor_row(n, pos, box, rc, i, src ? src + e : NULL, vec ? vec + 3 * e : NULL);
        if (row_ptr)
            row_ptr[i + 1] = (int32_t)e;
    }
    return e;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
