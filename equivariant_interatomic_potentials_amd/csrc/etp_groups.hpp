// etp_groups.hpp -- compile-time split of the path list into contiguous path
// groups, so that one wave's register accumulators for its group's output
// rows fit in the VGPR file, plus per-group derived ranges.
#pragma once
#include "etp_tables.hpp"

namespace etp {

constexpr int kMaxGroups = 32;

struct Groups {
    int n;
    int p0[kMaxGroups], p1[kMaxGroups];
};

// Greedy contiguous split: close a group when adding the next path would
// exceed max_rows output rows (a single path always fits).
constexpr Groups make_groups(const Table &T, int max_rows)
{
    Groups g{};
    int start = 0, rows = 0;
    for (int p = 0; p < T.P; ++p) {
        const int r = 2 * T.path[p].l3 + 1;
        if (rows > 0 && rows + r > max_rows) {
            g.p0[g.n] = start;
            g.p1[g.n] = p;
            ++g.n;
            start = p;
            rows = 0;
        }
        rows += r;
    }
    g.p0[g.n] = start;
    g.p1[g.n] = T.P;
    ++g.n;
    return g;
}

struct GroupInfo {
    int p0, p1, np;        // paths
    int pr0, pr1, npr;     // (m1, m3) pairs
    int stride;            // per-edge T stride in LDS (multiple of 4 floats)
    int row0, row1, nrow;  // output rows
    int xr0, xr1, nxr;     // x rows (all l1 present in the group)
};

constexpr GroupInfo group_info(const Table &T, const Groups &g, int k)
{
    GroupInfo gi{};
    gi.p0 = g.p0[k];
    gi.p1 = g.p1[k];
    gi.np = gi.p1 - gi.p0;
    gi.pr0 = T.path[gi.p0].pr0;
    gi.pr1 = T.path[gi.p1 - 1].pr1;
    gi.npr = gi.pr1 - gi.pr0;
    gi.stride = (gi.npr + 3) & ~3;
    gi.row0 = T.path[gi.p0].out_row;
    gi.row1 = T.path[gi.p1 - 1].out_row + 2 * T.path[gi.p1 - 1].l3 + 1;
    gi.nrow = gi.row1 - gi.row0;
    const int l1a = T.path[gi.p0].l1, l1b = T.path[gi.p1 - 1].l1;
    gi.xr0 = l1a * l1a;
    gi.xr1 = (l1b + 1) * (l1b + 1);
    gi.nxr = gi.xr1 - gi.xr0;
    return gi;
}

constexpr int max_stride(const Table &T, const Groups &g)
{
    int s = 0;
    for (int k = 0; k < g.n; ++k) {
        const int v = group_info(T, g, k).stride;
        s = v > s ? v : s;
    }
    return s;
}

// True when no earlier pair of the same path writes the same m3 (lets the
// first product of a per-m3 partial sum be a multiply instead of an FMA).
constexpr bool first_m3_in_path(const Table &T, int q)
{
    const Pair &pr = T.pair[q];
    for (int k = T.path[pr.path].pr0; k < q; ++k)
        if (T.pair[k].m3 == pr.m3)
            return false;
    return true;
}

// Same for m1 (partial sums indexed by the input row).
constexpr bool first_m1_in_path(const Table &T, int q)
{
    const Pair &pr = T.pair[q];
    for (int k = T.path[pr.path].pr0; k < q; ++k)
        if (T.pair[k].m1 == pr.m1)
            return false;
    return true;
}

// Source-side passes: contiguous path groups sized so that one edge's
// streamed operands (wmul weight rows per path + the G rows of the group's
// paths) plus the resident x rows and their accumulators fit the VGPR
// budget: cost = wmul * paths + G rows + 2 * x rows <= max_cost. A group may start
// inside an l1 block; the node rows of that l1 are then added to the rows
// the previous group stored.
struct SrcGroupInfo {
    int p0, p1, np;        // paths
    int ab0, ab1;          // (m1, m2) groups
    int xr0, xr1, nxr;     // x rows
    int gr0, gr1, ngr;     // G rows (out rows of the group's paths)
    bool shares_first_l1;  // an earlier group also touched the first l1
};

constexpr int src_cost(const Table &T, int p0, int p1, int wmul)
{
    const int l1a = T.path[p0].l1, l1b = T.path[p1 - 1].l1;
    const int xrows = (l1b + 1) * (l1b + 1) - l1a * l1a;
    const int grows = T.path[p1 - 1].out_row + 2 * T.path[p1 - 1].l3 + 1 - T.path[p0].out_row;
    return wmul * (p1 - p0) + grows + 2 * xrows;
}

constexpr Groups make_src_groups(const Table &T, int max_cost, int wmul)
{
    Groups g{};
    int start = 0;
    for (int p = 1; p <= T.P; ++p) {
        if (p == T.P || src_cost(T, start, p + 1, wmul) > max_cost) {
            g.p0[g.n] = start;
            g.p1[g.n] = p;
            ++g.n;
            start = p;
        }
    }
    return g;
}

constexpr SrcGroupInfo src_group_info(const Table &T, const Groups &g, int k)
{
    SrcGroupInfo gi{};
    gi.p0 = g.p0[k];
    gi.p1 = g.p1[k];
    gi.np = gi.p1 - gi.p0;
    gi.ab0 = T.path_ab0[gi.p0];
    gi.ab1 = T.path_ab0[gi.p1];
    const int l1a = T.path[gi.p0].l1, l1b = T.path[gi.p1 - 1].l1;
    gi.xr0 = l1a * l1a;
    gi.xr1 = (l1b + 1) * (l1b + 1);
    gi.nxr = gi.xr1 - gi.xr0;
    gi.gr0 = T.path[gi.p0].out_row;
    gi.gr1 = T.path[gi.p1 - 1].out_row + 2 * T.path[gi.p1 - 1].l3 + 1;
    gi.ngr = gi.gr1 - gi.gr0;
    gi.shares_first_l1 = gi.p0 > 0 && T.path[gi.p0 - 1].l1 == l1a;
    return gi;
}

// First (m1, m2) group of its path with this m1.
constexpr bool ab_first_m1(const Table &T, int g)
{
    const ABGroup &a = T.ab[g];
    for (int k = T.path_ab0[a.path]; k < g; ++k)
        if (T.ab[k].m1 == a.m1)
            return false;
    return true;
}

// First (m1, m2) group in [g0, g) that uses the SH index of g.
constexpr bool ab_first_b(const Table &T, int g0, int g)
{
    const ABGroup &a = T.ab[g];
    const int b = T.path[a.path].y_row + T.path[a.path].l2 + a.m2;
    for (int k = g0; k < g; ++k) {
        const ABGroup &o = T.ab[k];
        if (T.path[o.path].y_row + T.path[o.path].l2 + o.m2 == b)
            return false;
    }
    return true;
}

// Whether any (m1, m2) group in [g0, g1) uses SH index b.
constexpr bool ab_touches_b(const Table &T, int g0, int g1, int b)
{
    for (int k = g0; k < g1; ++k) {
        const ABGroup &o = T.ab[k];
        if (T.path[o.path].y_row + T.path[o.path].l2 + o.m2 == b)
            return true;
    }
    return false;
}

// Whether the VJP-of-VJP of path p takes fewer VALU operations per channel
// in the u / v order (per (m1, m2) group: K + 3; per m2 used: 7) than in the
// s / sd order (per group: K + 4; per m1: 7).
constexpr bool uv_cheaper(const Table &T, int p)
{
    const int nab = T.path_ab0[p + 1] - T.path_ab0[p];
    int nb = 0;
    for (int m = 0; m < 2 * T.path[p].l2 + 1; ++m)
        nb += ab_touches_b(T, T.path_ab0[p], T.path_ab0[p + 1], T.path[p].y_row + m) ? 1 : 0;
    return nab + 7 * (2 * T.path[p].l1 + 1) > 7 * nb;
}

// SH indices touched by the paths [p0, p1): [lo, hi).
constexpr int sh_lo(const Table &T, int p0, int p1)
{
    int lo = 1 << 20;
    for (int p = p0; p < p1; ++p)
        lo = T.path[p].y_row < lo ? T.path[p].y_row : lo;
    return lo;
}
constexpr int sh_hi(const Table &T, int p0, int p1)
{
    int hi = 0;
    for (int p = p0; p < p1; ++p) {
        const int h = T.path[p].y_row + 2 * T.path[p].l2 + 1;
        hi = h > hi ? h : hi;
    }
    return hi;
}

}  // namespace etp
