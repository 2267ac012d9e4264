// etp_neighbors.hip -- periodic neighbour list on the GPU: the
// destination-sorted CSR (sources ascending within a row) and the
// minimum-image bond vectors that the convolution walks ("edges per atom" in
// "How does FlashCart make equivariant interatomic potentials faster and more
// accurate?", section on the SPICE-MACE-OFF model).
//
// Contract (orthorhombic box, every side at least twice the cutoff):
//   q = p - L floor(p / L)                      wrapped position, per axis
//   d = q_j - q_i;  d = d - L rint(d / L)        minimum image, per axis
//   r2 = fma(dz, dz, fma(dy, dy, dx * dx))
//   edge (i <- j) iff j != i and r2 < rc * rc, all in float32;  vec = d.
// The cutoff decision turns floating point into integers, so it is taken in
// float32 with every operation spelled out (fused multiply-adds where
// written, correctly rounded division, round-half-even rint): any
// implementation of the contract produces the same edges bit for bit.
//
// Steps (a cell list, then two sweeps over it):
//   1. bin: wrap every atom, give it a cell of side >= rc (1 + 2^-10) and a
//      rank in that cell (integer atomics; the ranks depend on scheduling,
//      nothing downstream does);
//   2. scan the cell counts into cell offsets; scatter the wrapped positions
//      (and atom ids) into cell order;
//   3. count: one wave per atom (atoms in cell order, so neighbouring waves
//      read the same cells); the 27 (fewer when a box side holds fewer than
//      3 cells) neighbouring cells are flattened into one candidate range,
//      64 candidates per step, and every hit is counted with a ballot;
//   4. scan the counts into row_ptr;                  (end of the count call)
//   5. fill: the same sweep gathers each row's sources at slots from ballot
//      prefix counts (in LDS for rows up to kNlRowCap, else unordered in src);
//   6. sort the row by source id (rank by counting: the ids in a row are
//      distinct) -- in the fill for rows in LDS, else in nl_sort_kernel
//      through the row's own part of the vec buffer, free until step 7;
//   7. vec of every edge from the wrapped positions, in the contract's
//      arithmetic (in the fill, or in nl_vec_kernel for long rows).
// Cells have side >= rc (1 + 2^-10), so two atoms closer than the cutoff sit
// in the same or adjacent cells even after the float32 rounding of the cell
// index (an error of a few 1e-5 cell sides for up to kNlMaxCellsAxis cells
// per axis).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "etp_device.hpp"

namespace etp {

hipError_t launch_nl_fill_int(int *p, int64_t n, int v, hipStream_t stream);
hipError_t launch_nl_counts_to_offsets(int *ptr, int64_t n, int *bsum, hipStream_t stream);
int64_t scan_bsum_ints(int64_t n);

constexpr int kNlMaxCellsAxis = 128;
constexpr int kNlRowCap = 1024;  // row length sorted in LDS (per wave)

struct NlGeom {
    float L[3];   // box sides
    float f[3];   // cells per unit length (binning scale)
    int nc[3];    // cells per axis
    int no[3];    // neighbour offsets per axis: min(nc, 3)
    float rc2;    // rc * rc in float32
    int ncell;
};

struct NlWork {
    int *cell_start;  // [ncell + 1]
    int *cell_rank;   // [n]: (cell, rank within cell)
    int *cell_of;     // [n]
    float4 *qa;       // [n]: wrapped positions by atom id
    float4 *cq;       // [n]: wrapped positions in cell order, w = atom id bits
    int *bsum;        // scan tile totals
    int *bad;         // [1]: rows whose fill count differs from row_ptr
};

__device__ __forceinline__ float nl_wrap(float p, float L) { return __builtin_fmaf(-L, floorf(p / L), p); }

// d - L rint(d / L) for d = q_j - q_i of wrapped positions (|d| <= L). The
// division is taken only where its rounding can matter: for |d| <= L/4 the
// correctly rounded quotient lies in [-1/4, 1/4] and rint gives 0; for |d| >=
// fl(3L/4) it lies in (1/2, 1] and rint gives sign(d); in between the
// quotient is formed. The result is bit-identical to the formula as written
// (also for d = 0: both give +0), and most candidates of a cell list take the
// first branch.
__device__ __forceinline__ float nl_image(float d, float L)
{
    const float a = fabsf(d);
    float k;
    if (a <= 0.25f * L)
        k = 0.f;
    else if (a >= 0.75f * L)
        k = copysignf(1.f, d);
    else
        k = rintf(d / L);
    return __builtin_fmaf(-L, k, d);
}

__device__ __forceinline__ int nl_axis_cell(float q, float f, int nc)
{
    const int c = static_cast<int>(floorf(q * f));
    return c < 0 ? 0 : (c >= nc ? nc - 1 : c);
}

__device__ __forceinline__ int nl_cell_id(const NlGeom &g, int cx, int cy, int cz)
{
    return (cz * g.nc[1] + cy) * g.nc[0] + cx;
}

// step 1: wrap, cell, rank within the cell
__global__ void __launch_bounds__(256) nl_bin_kernel(int n, const float *__restrict__ pos, const NlGeom g, NlWork w)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const float qx = nl_wrap(pos[3 * static_cast<int64_t>(i)], g.L[0]);
    const float qy = nl_wrap(pos[3 * static_cast<int64_t>(i) + 1], g.L[1]);
    const float qz = nl_wrap(pos[3 * static_cast<int64_t>(i) + 2], g.L[2]);
    const int c = nl_cell_id(g, nl_axis_cell(qx, g.f[0], g.nc[0]), nl_axis_cell(qy, g.f[1], g.nc[1]),
                             nl_axis_cell(qz, g.f[2], g.nc[2]));
    w.qa[i] = make_float4(qx, qy, qz, 0.f);
    w.cell_of[i] = c;
    w.cell_rank[i] = atomicAdd(&w.cell_start[c + 1], 1);
}

// step 2b: positions into cell order
__global__ void __launch_bounds__(256) nl_scatter_kernel(int n, NlWork w)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    const float4 q = w.qa[i];
    w.cq[w.cell_start[w.cell_of[i]] + w.cell_rank[i]] = make_float4(q.x, q.y, q.z, __int_as_float(i));
}

// steps 3 and 5: one wave per atom, atoms taken in cell order. The fill
// keeps a row of up to kNlRowCap sources in LDS, ranks it there and writes
// src and vec in order (steps 5-7 in one pass); a longer row is written
// unordered and left to nl_sort_kernel / nl_vec_kernel.
template <bool FILL>
__global__ void __launch_bounds__(256) nl_sweep_kernel(int n, const NlGeom g, NlWork w, int *__restrict__ row_ptr,
                                                       int *__restrict__ src, float *__restrict__ vec)
{
    __shared__ int cstart_s[4][32];
    __shared__ int cpre_s[4][32];
    __shared__ int4 buf_s[FILL ? 4 : 1][FILL ? kNlRowCap / 4 + 1 : 1];
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int slot = blockIdx.x * 4 + wv;
    if (slot >= n)
        return;
    int *cstart = cstart_s[wv], *cpre = cpre_s[wv];
    const float4 me = w.cq[slot];
    const int i = __float_as_int(me.w);
    const int cx = nl_axis_cell(me.x, g.f[0], g.nc[0]), cy = nl_axis_cell(me.y, g.f[1], g.nc[1]),
              cz = nl_axis_cell(me.z, g.f[2], g.nc[2]);

    // the neighbouring cells, one per lane, flattened into one range
    const int K = g.no[0] * g.no[1] * g.no[2];
    int cnt = 0, start = 0;
    if (lane < K) {
        const int ox = lane % g.no[0], oy = (lane / g.no[0]) % g.no[1], oz = lane / (g.no[0] * g.no[1]);
        const int x = (cx + ox - (g.no[0] == 3) + g.nc[0]) % g.nc[0];
        const int y = (cy + oy - (g.no[1] == 3) + g.nc[1]) % g.nc[1];
        const int z = (cz + oz - (g.no[2] == 3) + g.nc[2]) % g.nc[2];
        const int c = nl_cell_id(g, x, y, z);
        start = w.cell_start[c];
        cnt = w.cell_start[c + 1] - start;
    }
    int incl = cnt;
    for (int s = 1; s < 32; s <<= 1) {
        const int t = __shfl_up(incl, s, 64);
        if (lane >= s)
            incl += t;
    }
    const int total = __shfl(incl, 31, 64);  // K <= 27: lanes 27..63 hold no cells
    if (lane < K) {
        cstart[lane] = start;
        cpre[lane] = incl - cnt;  // exclusive prefix
    }
    wave_sync_lds();

    int base = 0, lim = 0;
    if constexpr (FILL) {
        base = row_ptr[i];
        lim = row_ptr[i + 1] - base;
    }
    const bool inl = FILL && lim <= kNlRowCap;  // this row is ordered in LDS
    int *buf = reinterpret_cast<int *>(buf_s[FILL ? wv : 0]);
    // this lane's candidate v in cell order: its cell is the last t with
    // cpre[t] <= v (cells may be empty); t only moves forward
    int t = 0, found = 0;
    auto locate = [&](int v) {
        while (t + 1 < K && cpre[t + 1] <= v)
            ++t;
        return cstart[t] + (v - cpre[t]);
    };
    // one step of look-ahead: the next step's candidate is loaded before this
    // step's test
    float4 nxt = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane < total)
        nxt = w.cq[locate(lane)];
    for (int v0 = 0; v0 < total; v0 += 64) {
        const int v = v0 + lane;
        const float4 o = nxt;
        if (v + 64 < total)
            nxt = w.cq[locate(v + 64)];
        bool hit = false;
        int j = 0;
        if (v < total) {
            j = __float_as_int(o.w);
            const float dx = nl_image(o.x - me.x, g.L[0]);
            const float dy = nl_image(o.y - me.y, g.L[1]);
            const float dz = nl_image(o.z - me.z, g.L[2]);
            const float r2 = __builtin_fmaf(dz, dz, __builtin_fmaf(dy, dy, dx * dx));
            hit = (j != i) && (r2 < g.rc2);
        }
        const uint64_t m = __ballot(hit);
        if constexpr (FILL) {
            const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
            const int k = found + below;
            if (hit && k < lim) {
                if (inl)
                    buf[k] = j;
                else
                    src[base + k] = j;
            }
        }
        found += __popcll(m);
    }
    if constexpr (FILL) {
        const int have = found < lim ? found : lim;
        if (inl) {
            // rank by counting (the ids of a row are distinct), four ids per
            // LDS read; the padding after the row never counts
            if (lane < 4)
                buf[have + lane] = 0x7FFFFFFF;
            wave_sync_lds();
            const int4 *b4 = buf_s[wv];
            const int nq = (have + 3) >> 2;
            for (int k = lane; k < have; k += 64) {
                const int v = buf[k];
                int r = 0;
                for (int q = 0; q < nq; ++q) {
                    const int4 b = b4[q];
                    r += (b.x < v) + (b.y < v) + (b.z < v) + (b.w < v);
                }
                const float4 o = w.qa[v];
                float *ve = vec + 3 * (static_cast<int64_t>(base) + r);
                src[base + r] = v;
                ve[0] = nl_image(o.x - me.x, g.L[0]);
                ve[1] = nl_image(o.y - me.y, g.L[1]);
                ve[2] = nl_image(o.z - me.z, g.L[2]);
            }
        }
        // positions changed since the count: pad the row and flag it
        for (int k = have + lane; k < lim; k += 64) {
            src[base + k] = -1;
            if (inl) {
                float *ve = vec + 3 * (static_cast<int64_t>(base) + k);
                ve[0] = ve[1] = ve[2] = __builtin_nanf("");
            }
        }
        if (lane == 0 && found != lim)
            atomicAdd(w.bad, 1);
    } else {
        if (lane == 0)
            row_ptr[i + 1] = found;
    }
}

// step 6 for rows longer than kNlRowCap: sort by source id, one wave per
// row, rank by counting through scratch in the row's own part of the vec
// buffer (3 len floats, not yet written; other rows' vec is never touched).
__global__ void __launch_bounds__(256) nl_sort_kernel(int n, const int *__restrict__ row_ptr, int *__restrict__ src,
                                                      int *__restrict__ scratch)
{
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + wave_id();
    if (i >= n)
        return;
    const int s = row_ptr[i], len = row_ptr[i + 1] - s;
    if (len <= kNlRowCap)
        return;  // ordered by the fill
    int *buf = scratch + 3 * static_cast<int64_t>(s);
    for (int k = lane; k < len; k += 64)
        buf[k] = src[s + k];
    __threadfence();  // the wave's stores complete before its loads, which miss L1
    for (int k = lane; k < len; k += 64) {
        const int v = buf[k];
        int r = 0;
        for (int q = 0; q < len; ++q)
            r += buf[q] < v;
        src[s + r] = v;
    }
}

// step 7 for rows longer than kNlRowCap: vec of every edge; one wave per row.
__global__ void __launch_bounds__(256) nl_vec_kernel(int n, const NlGeom g, const float4 *__restrict__ qa,
                                                     const int *__restrict__ row_ptr, const int *__restrict__ src,
                                                     float *__restrict__ vec)
{
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + wave_id();
    if (i >= n)
        return;
    const int s = row_ptr[i], e1 = row_ptr[i + 1];
    if (e1 - s <= kNlRowCap)
        return;  // written by the fill
    const float4 me = qa[i];
    for (int e = s + lane; e < e1; e += 64) {
        const int j = src[e];
        float dx = __builtin_nanf(""), dy = dx, dz = dx;
        if (static_cast<unsigned>(j) < static_cast<unsigned>(n)) {
            const float4 o = qa[j];
            dx = nl_image(o.x - me.x, g.L[0]);
            dy = nl_image(o.y - me.y, g.L[1]);
            dz = nl_image(o.z - me.z, g.L[2]);
        }
        float *ve = vec + 3 * static_cast<int64_t>(e);
        ve[0] = dx;
        ve[1] = dy;
        ve[2] = dz;
    }
}

// ------------------------------------------------------------------ host

static NlGeom nl_geom(const float *box, float rc)
{
    NlGeom g{};
    for (int a = 0; a < 3; ++a) {
        g.L[a] = box[a];
        int nc = static_cast<int>(std::floor(static_cast<double>(box[a]) / (static_cast<double>(rc) * (1.0 + 1.0 / 1024))));
        nc = nc < 1 ? 1 : (nc > kNlMaxCellsAxis ? kNlMaxCellsAxis : nc);
        g.nc[a] = nc;
        g.no[a] = nc < 3 ? nc : 3;
        g.f[a] = static_cast<float>(nc / static_cast<double>(box[a]));
    }
    g.rc2 = rc * rc;
    g.ncell = g.nc[0] * g.nc[1] * g.nc[2];
    return g;
}

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t neighbor_workspace_bytes(int n, const float *box, float rc)
{
    const NlGeom g = nl_geom(box, rc);
    const int64_t nb = scan_bsum_ints(n > g.ncell ? n : g.ncell);
    return align256(sizeof(int) * (g.ncell + 1)) + 2 * align256(sizeof(int) * static_cast<size_t>(n)) +
           2 * align256(sizeof(float4) * static_cast<size_t>(n)) + align256(sizeof(int) * (nb + 1)) + 256;
}

static NlWork nl_carve(void *ws, int n, const NlGeom &g)
{
    char *p = static_cast<char *>(ws);
    NlWork w;
    auto take = [&](size_t b) {
        char *q = p;
        p += align256(b);
        return q;
    };
    w.cell_start = reinterpret_cast<int *>(take(sizeof(int) * (g.ncell + 1)));
    w.cell_rank = reinterpret_cast<int *>(take(sizeof(int) * static_cast<size_t>(n)));
    w.cell_of = reinterpret_cast<int *>(take(sizeof(int) * static_cast<size_t>(n)));
    w.qa = reinterpret_cast<float4 *>(take(sizeof(float4) * static_cast<size_t>(n)));
    w.cq = reinterpret_cast<float4 *>(take(sizeof(float4) * static_cast<size_t>(n)));
    w.bad = reinterpret_cast<int *>(take(sizeof(int)));
    w.bsum = reinterpret_cast<int *>(p);
    return w;
}

// steps 1-2
static hipError_t nl_bin(int n, const float *pos, const NlGeom &g, const NlWork &w, hipStream_t stream)
{
    hipError_t e = launch_nl_fill_int(w.cell_start, g.ncell + 1, 0, stream);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(nl_bin_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, n, pos, g, w);
    if ((e = launch_nl_counts_to_offsets(w.cell_start, g.ncell, w.bsum, stream)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(nl_scatter_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, n, w);
    return hipGetLastError();
}

hipError_t launch_neighbor_count(int n, const float *pos, const float *box, float rc, int *row_ptr, void *ws,
                                 hipStream_t stream)
{
    hipError_t e = launch_nl_fill_int(row_ptr, 1, 0, stream);
    if (e != hipSuccess || n == 0)
        return e;
    const NlGeom g = nl_geom(box, rc);
    const NlWork w = nl_carve(ws, n, g);
    if ((e = nl_bin(n, pos, g, w, stream)) != hipSuccess)
        return e;
    hipLaunchKernelGGL(nl_sweep_kernel<false>, dim3((n + 3) / 4), dim3(256), 0, stream, n, g, w, row_ptr,
                       static_cast<int *>(nullptr), static_cast<float *>(nullptr));
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return launch_nl_counts_to_offsets(row_ptr, n, w.bsum, stream);
}

hipError_t launch_neighbor_fill(int n, const float *pos, const float *box, float rc, const int *row_ptr,
                                int64_t n_edges, int *src, float *vec, void *ws, int **bad, hipStream_t stream)
{
    const NlGeom g = nl_geom(box, rc);
    const NlWork w = nl_carve(ws, n, g);
    *bad = w.bad;
    hipError_t e = launch_nl_fill_int(w.bad, 1, 0, stream);
    if (e != hipSuccess || n == 0)
        return e;
    if ((e = nl_bin(n, pos, g, w, stream)) != hipSuccess)
        return e;
    if (n_edges == 0)
        return hipSuccess;
    int *rp = const_cast<int *>(row_ptr);  // read only in the fill sweep
    hipLaunchKernelGGL(nl_sweep_kernel<true>, dim3((n + 3) / 4), dim3(256), 0, stream, n, g, w, rp, src, vec);
    hipLaunchKernelGGL(nl_sort_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, n, row_ptr, src,
                       reinterpret_cast<int *>(vec));
    hipLaunchKernelGGL(nl_vec_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, n, g, w.qa, row_ptr, src, vec);
    return hipGetLastError();
}

}  // namespace etp
