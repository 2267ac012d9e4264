// etp_tables.hpp -- compile-time path table and sparse real Clebsch-Gordan
// table for the edge tensor-product convolution.
//
// The tensor product couples source-node irreps (l1) with the bond-vector
// spherical harmonics (l2) into outputs (l3) through Wigner 3-j coefficients
// kept in a compressed sparse form ("High-performance training and inference
// for deep equivariant interatomic potentials", review page, section
// "Proposed method"). The pages give no formulas; this file evaluates the
// textbook ones:
//   * Wigner 3-j symbols from Racah's single-sum formula;
//   * complex CG <j1 m1 j2 m2 | J M> = (-1)^(j1-j2+M) sqrt(2J+1) (j1 j2 J; m1 m2 -M);
//   * the real basis r_{l,mu}: mu>0 -> (|l,-mu> + (-1)^mu |l,mu>)/sqrt2,
//     mu=0 -> |l,0>, mu<0 (k=-mu) -> i(|l,-k> - (-1)^k |l,k>)/sqrt2; the real
//     coupling is Re of the transformed tensor for even l1+l2+l3, Im for odd;
//   * paths (l1, l2, l3) in lexicographic order with |l1-l2| <= l3 <=
//     min(l1+l2, L), every one kept (SO(3), no parity);
//   * entries with |C| > 1e-12, ordered by (m1, m2, m3).
// Everything is constexpr, so device code folds the coefficients into
// immediates and the host plan returns exactly the same values.
#pragma once
#include <cstdint>

namespace etp {

constexpr int kLMax = 4;

// ---------------------------------------------------------------- math ----
constexpr double cx_sqrt(double a)
{
    // Newton's iteration from above; it decreases monotonically to within an
    // ulp of the root and stops when it no longer decreases.
    if (a <= 0.0)
        return 0.0;
    double x = a < 1.0 ? 1.0 : a;
    for (int i = 0; i < 400; ++i) {
        double nx = 0.5 * (x + a / x);
        if (nx >= x)
            break;
        x = nx;
    }
    return x;
}

constexpr double cx_fact(int n)
{
    double r = 1.0;
    for (int i = 2; i <= n; ++i)
        r *= i;
    return r;
}

constexpr int cx_abs(int a) { return a < 0 ? -a : a; }
constexpr int cx_min(int a, int b) { return a < b ? a : b; }
constexpr int cx_max(int a, int b) { return a > b ? a : b; }
constexpr double cx_fabs(double a) { return a < 0 ? -a : a; }
constexpr double cx_sign_pow(int n) { return (n % 2 == 0) ? 1.0 : -1.0; }  // (-1)^n, n may be < 0

// Wigner 3-j symbol (j1 j2 j3; m1 m2 m3), Racah's formula.
constexpr double wigner3j(int j1, int j2, int j3, int m1, int m2, int m3)
{
    if (m1 + m2 + m3 != 0)
        return 0.0;
    if (j3 < cx_abs(j1 - j2) || j3 > j1 + j2)
        return 0.0;
    if (cx_abs(m1) > j1 || cx_abs(m2) > j2 || cx_abs(m3) > j3)
        return 0.0;
    const double tri = cx_fact(j1 + j2 - j3) * cx_fact(j1 - j2 + j3) * cx_fact(-j1 + j2 + j3) /
                       cx_fact(j1 + j2 + j3 + 1);
    const double mf = cx_fact(j1 + m1) * cx_fact(j1 - m1) * cx_fact(j2 + m2) * cx_fact(j2 - m2) *
                      cx_fact(j3 + m3) * cx_fact(j3 - m3);
    const int kmin = cx_max(0, cx_max(j2 - j3 - m1, j1 - j3 + m2));
    const int kmax = cx_min(j1 + j2 - j3, cx_min(j1 - m1, j2 + m2));
    double s = 0.0;
    for (int k = kmin; k <= kmax; ++k) {
        const double den = cx_fact(k) * cx_fact(j3 - j2 + k + m1) * cx_fact(j3 - j1 + k - m2) *
                           cx_fact(j1 + j2 - j3 - k) * cx_fact(j1 - k - m1) * cx_fact(j2 - k + m2);
        s += cx_sign_pow(k) / den;
    }
    return cx_sign_pow(j1 - j2 - m3) * cx_sqrt(tri * mf) * s;
}

constexpr double cg_complex(int j1, int m1, int j2, int m2, int J, int M)
{
    return cx_sign_pow(j1 - j2 + M) * cx_sqrt(2.0 * J + 1.0) * wigner3j(j1, j2, J, m1, m2, -M);
}

struct cplx {
    double re, im;
};
constexpr cplx cmul(cplx a, cplx b) { return {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re}; }
constexpr cplx cconj(cplx a) { return {a.re, -a.im}; }

// The (at most two) complex components m of real basis vector mu, with the
// coefficient of |l, m> in r_{l,mu}.
struct basis_terms {
    int n;
    int m[2];
    cplx c[2];
};
constexpr basis_terms real_basis_terms(int mu)
{
    const double h = 0.70710678118654752440;
    basis_terms t{};
    if (mu == 0) {
        t.n = 1;
        t.m[0] = 0;
        t.c[0] = {1.0, 0.0};
    } else if (mu > 0) {
        t.n = 2;
        t.m[0] = -mu;
        t.c[0] = {h, 0.0};
        t.m[1] = mu;
        t.c[1] = {cx_sign_pow(mu) * h, 0.0};
    } else {
        const int k = -mu;
        t.n = 2;
        t.m[0] = -k;
        t.c[0] = {0.0, h};
        t.m[1] = k;
        t.c[1] = {0.0, -cx_sign_pow(k) * h};
    }
    return t;
}

// Real coupling coefficient for real indices (a, b, c) = (mu1, mu2, mu3).
constexpr double cg_real(int l1, int l2, int l3, int a, int b, int c)
{
    const basis_terms A = real_basis_terms(a), B = real_basis_terms(b), Cc = real_basis_terms(c);
    cplx s{0.0, 0.0};
    for (int i = 0; i < A.n; ++i)
        for (int j = 0; j < B.n; ++j)
            for (int k = 0; k < Cc.n; ++k) {
                if (A.m[i] + B.m[j] != Cc.m[k])
                    continue;
                const double g = cg_complex(l1, A.m[i], l2, B.m[j], l3, Cc.m[k]);
                if (g == 0.0)
                    continue;
                cplx t = cmul(cmul(Cc.c[k], cconj(A.c[i])), cconj(B.c[j]));
                s.re += t.re * g;
                s.im += t.im * g;
            }
    return ((l1 + l2 + l3) % 2 == 0) ? s.re : s.im;
}

// --------------------------------------------------------------- tables ---
struct Path {
    int l1, l2, l3;
    int nz0, nz1;      // CG entries [nz0, nz1)
    int pr0, pr1;      // (m1, m3) pairs [pr0, pr1)
    int out_row;       // first output row of this path (rows = 2 l3 + 1)
    int x_row;         // first x row of l1: l1*l1
    int y_row;         // first SH index of l2: l2*l2
};

struct Entry {
    int m1, m2, m3;    // signed m values
    double val;        // float64 coefficient
    float fval;        // round-to-nearest float32 of val
    int pair;          // index of its (path, m1, m3) pair
};

struct Pair {
    int path;
    int m1, m3;        // signed
    int t0, t1;        // entry indices in pair_entries [t0, t1)
};

// Entries of one path grouped by (m1, m2): the contraction over m3 used by
// the source-side passes.
struct ABGroup {
    int path;
    int m1, m2;        // signed
    int t0, t1;        // entry indices in ab_entries [t0, t1)
};

constexpr int kMaxPaths = 65, kMaxNnz = 2052, kMaxPairs = 1724;

struct Table {
    int L;
    int P, nnz, npair;
    int din_rows, dsh, dout_rows;
    Path path[kMaxPaths];
    Entry nz[kMaxNnz];
    Pair pair[kMaxPairs];
    int pair_entries[kMaxNnz];  // entry indices grouped by pair, (m2) ascending within a pair
    int nab;
    ABGroup ab[kMaxPairs];
    int ab_entries[kMaxNnz];    // entry indices grouped by (path, m1, m2), m3 ascending
    int path_ab0[kMaxPaths + 1];
};

constexpr Table make_table(int L)
{
    Table T{};
    T.L = L;
    T.din_rows = (L + 1) * (L + 1);
    T.dsh = (L + 1) * (L + 1);
    int P = 0, nnz = 0, npair = 0, row = 0, pe = 0;
    for (int l1 = 0; l1 <= L; ++l1)
        for (int l2 = 0; l2 <= L; ++l2)
            for (int l3 = cx_abs(l1 - l2); l3 <= cx_min(l1 + l2, L); ++l3) {
                Path &p = T.path[P];
                p.l1 = l1;
                p.l2 = l2;
                p.l3 = l3;
                p.out_row = row;
                p.x_row = l1 * l1;
                p.y_row = l2 * l2;
                row += 2 * l3 + 1;
                p.nz0 = nnz;
                // entries in (m1, m2, m3) order; the real selection rule
                // |m3| in {|m1|+|m2|, ||m1|-|m2||} prunes the candidates
                for (int a = -l1; a <= l1; ++a)
                    for (int b = -l2; b <= l2; ++b)
                        for (int c = -l3; c <= l3; ++c) {
                            const int aa = cx_abs(a), ab = cx_abs(b), ac = cx_abs(c);
                            if (ac != aa + ab && ac != cx_abs(aa - ab))
                                continue;
                            const double v = cg_real(l1, l2, l3, a, b, c);
                            if (cx_fabs(v) <= 1e-12)
                                continue;
                            Entry &e = T.nz[nnz++];
                            e.m1 = a;
                            e.m2 = b;
                            e.m3 = c;
                            e.val = v;
                            e.fval = static_cast<float>(v);
                            e.pair = -1;
                        }
                p.nz1 = nnz;
                // group entries of this path by (m1, m3)
                p.pr0 = npair;
                for (int a = -l1; a <= l1; ++a)
                    for (int c = -l3; c <= l3; ++c) {
                        int cnt = 0;
                        for (int t = p.nz0; t < p.nz1; ++t)
                            if (T.nz[t].m1 == a && T.nz[t].m3 == c)
                                ++cnt;
                        if (!cnt)
                            continue;
                        Pair &q = T.pair[npair];
                        q.path = P;
                        q.m1 = a;
                        q.m3 = c;
                        q.t0 = pe;
                        for (int t = p.nz0; t < p.nz1; ++t)
                            if (T.nz[t].m1 == a && T.nz[t].m3 == c) {
                                T.pair_entries[pe++] = t;
                                T.nz[t].pair = npair;
                            }
                        q.t1 = pe;
                        ++npair;
                    }
                p.pr1 = npair;
                ++P;
            }
    T.P = P;
    T.nnz = nnz;
    T.npair = npair;
    T.dout_rows = row;
    // (m1, m2) groups: entries are already in (m1, m2, m3) order within a path
    int nab = 0, ae = 0;
    for (int p = 0; p < P; ++p) {
        T.path_ab0[p] = nab;
        for (int t = T.path[p].nz0; t < T.path[p].nz1; ++t) {
            const bool fresh = (t == T.path[p].nz0) || T.nz[t - 1].m1 != T.nz[t].m1 ||
                               T.nz[t - 1].m2 != T.nz[t].m2;
            if (fresh) {
                if (nab > 0 && T.ab[nab - 1].path == p)
                    T.ab[nab - 1].t1 = ae;
                ABGroup &g = T.ab[nab++];
                g.path = p;
                g.m1 = T.nz[t].m1;
                g.m2 = T.nz[t].m2;
                g.t0 = ae;
            }
            T.ab_entries[ae++] = t;
        }
        if (nab > 0 && T.ab[nab - 1].path == p)
            T.ab[nab - 1].t1 = ae;
    }
    T.path_ab0[P] = nab;
    T.nab = nab;
    return T;
}

// The table of l_max = L (a namespace-scope constant, usable from device
// lambdas without capture).
template <int L>
inline constexpr Table kTab = make_table(L);

// Runtime access (host): a pointer to the table of l_max = L.
const Table *table_for(int L);

}  // namespace etp
