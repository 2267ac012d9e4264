// Host check of the library's plan-table code under AddressSanitizer and
// UndefinedBehaviorSanitizer: make_table(L) is evaluated at run time (a
// volatile l_max keeps the compiler from folding it), with every array index
// and integer operation checked, and compared field by field with the
// compile-time table the kernels and the plan use. Built and run by
// tests/test_host_sanitizers.py (g++, no GPU code).
#include <cstdio>
#include <cstring>

#include "etp_tables.hpp"

namespace {

const etp::Table *compiled(int L)
{
    switch (L) {
    case 0: return &etp::kTab<0>;
    case 1: return &etp::kTab<1>;
    case 2: return &etp::kTab<2>;
    case 3: return &etp::kTab<3>;
    default: return &etp::kTab<4>;
    }
}

bool same_double(double a, double b) { return std::memcmp(&a, &b, sizeof a) == 0; }
bool same_float(float a, float b) { return std::memcmp(&a, &b, sizeof a) == 0; }

int compare(const etp::Table &a, const etp::Table &b)
{
    int bad = 0;
    bad += a.L != b.L || a.P != b.P || a.nnz != b.nnz || a.npair != b.npair || a.nab != b.nab;
    bad += a.din_rows != b.din_rows || a.dsh != b.dsh || a.dout_rows != b.dout_rows;
    for (int p = 0; p < a.P; ++p) {
        const etp::Path &x = a.path[p], &y = b.path[p];
        bad += x.l1 != y.l1 || x.l2 != y.l2 || x.l3 != y.l3 || x.nz0 != y.nz0 || x.nz1 != y.nz1 ||
               x.pr0 != y.pr0 || x.pr1 != y.pr1 || x.out_row != y.out_row || x.x_row != y.x_row ||
               x.y_row != y.y_row;
        bad += a.path_ab0[p] != b.path_ab0[p];
    }
    bad += a.path_ab0[a.P] != b.path_ab0[b.P];
    for (int t = 0; t < a.nnz; ++t) {
        const etp::Entry &x = a.nz[t], &y = b.nz[t];
        bad += x.m1 != y.m1 || x.m2 != y.m2 || x.m3 != y.m3 || x.pair != y.pair;
        bad += !same_double(x.val, y.val) || !same_float(x.fval, y.fval);
        bad += a.pair_entries[t] != b.pair_entries[t] || a.ab_entries[t] != b.ab_entries[t];
    }
    for (int q = 0; q < a.npair; ++q) {
        const etp::Pair &x = a.pair[q], &y = b.pair[q];
        bad += x.path != y.path || x.m1 != y.m1 || x.m3 != y.m3 || x.t0 != y.t0 || x.t1 != y.t1;
    }
    for (int g = 0; g < a.nab; ++g) {
        const etp::ABGroup &x = a.ab[g], &y = b.ab[g];
        bad += x.path != y.path || x.m1 != y.m1 || x.m2 != y.m2 || x.t0 != y.t0 || x.t1 != y.t1;
    }
    return bad;
}

}  // namespace

int main()
{
    static etp::Table rt;  // (large: kept off the stack)
    int bad = 0;
    for (int L = 0; L <= etp::kLMax; ++L) {
        volatile int l = L;
        rt = etp::make_table(l);
        const int d = compare(rt, *compiled(L));
        std::printf("l_max=%d P=%d nnz=%d pairs=%d mismatches=%d\n", L, rt.P, rt.nnz, rt.npair, d);
        bad += d;
    }
    return bad == 0 ? 0 : 1;
}
