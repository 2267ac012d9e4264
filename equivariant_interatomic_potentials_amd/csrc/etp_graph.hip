// etp_graph.hip -- graph preparation: the stable transpose of a
// destination-sorted CSR edge list (source offsets, edge ids grouped by
// source in edge-id order, and each such edge's destination), plus an
// optional validity check of the CSR.
//
// The neighbour list is the structure the convolution walks ("edges per
// atom" in "How does FlashCart make equivariant interatomic potentials faster
// and more accurate?", section on the SPICE-MACE-OFF model); the source-side
// passes of the VJP need it grouped by source.
//
// Steps (all integer, bit-exact and deterministic):
//   1. counts[src[e]]++ with integer atomics (the totals do not depend on
//      the order of the increments);
//   2. exclusive scan of the counts into src_ptr (tile scan + scan of tile
//      totals + offsets);
//   3. each edge takes a slot in its source's segment with an atomic
//      cursor (arbitrary order), then every segment is sorted by edge id
//      (LDS bitonic sort, or rank-by-counting for segments longer than the
//      LDS tile), which makes the result independent of the atomic order;
//   4. perm_dst[k] = the row of perm[k], by binary search in row_ptr.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <mutex>

namespace etp {

constexpr int kScanThreads = 256, kScanItems = 8, kScanTile = kScanThreads * kScanItems;
constexpr int kSortCap = 2048;

// The fill and scan kernels serve several callers; TAG (kTagTranspose,
// kTagNeighbors) only gives each caller its own kernel names, so that a
// kernel trace attributes their time to the right step.
constexpr int kTagTranspose = 0, kTagNeighbors = 1;

template <int TAG>
__global__ void __launch_bounds__(256) fill_kernel(int *__restrict__ p, int64_t n, int v)
{
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        p[i] = v;
}

__global__ void __launch_bounds__(256) hist_kernel(int64_t E, const int *__restrict__ src, int *__restrict__ counts)
{
    for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < E;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x)
        atomicAdd(&counts[src[e]], 1);
}

// Inclusive scan of the 256 thread totals of a block (returns the inclusive
// value of this thread; *total receives the block total).
__device__ int block_inclusive_scan(int v, int *total)
{
    __shared__ int wsum[kScanThreads / 64];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d, 64);
        if (lane >= d)
            v += t;
    }
    if (lane == 63)
        wsum[wid] = v;
    __syncthreads();
    int off = 0, tot = 0;
    for (int k = 0; k < kScanThreads / 64; ++k) {
        if (k < wid)
            off += wsum[k];
        tot += wsum[k];
    }
    __syncthreads();
    *total = tot;
    return v + off;
}

// In-place inclusive scan of each tile of a[0, n); tile totals to bsum.
template <int TAG>
__global__ void __launch_bounds__(kScanThreads) scan_tiles_kernel(int *__restrict__ a, int64_t n, int *__restrict__ bsum)
{
    const int64_t base = blockIdx.x * static_cast<int64_t>(kScanTile) + threadIdx.x * kScanItems;
    int v[kScanItems];
    int run = 0;
    for (int k = 0; k < kScanItems; ++k) {
        v[k] = (base + k < n) ? a[base + k] : 0;
        run += v[k];
        v[k] = run;
    }
    int total;
    const int incl = block_inclusive_scan(run, &total);
    const int excl = incl - run;
    for (int k = 0; k < kScanItems; ++k)
        if (base + k < n)
            a[base + k] = v[k] + excl;
    if (threadIdx.x == 0)
        bsum[blockIdx.x] = total;
}

// Single-block inclusive scan of b[0, n) in place.
template <int TAG>
__global__ void __launch_bounds__(kScanThreads) scan_single_kernel(int *__restrict__ b, int64_t n)
{
    int carry = 0;
    for (int64_t base = 0; base < n; base += kScanThreads) {
        const int64_t i = base + threadIdx.x;
        const int v = i < n ? b[i] : 0;
        int total;
        const int incl = block_inclusive_scan(v, &total);
        if (i < n)
            b[i] = incl + carry;
        carry += total;
    }
}

template <int TAG>
__global__ void __launch_bounds__(kScanThreads) add_offsets_kernel(int *__restrict__ a, int64_t n,
                                                                   const int *__restrict__ bsum)
{
    if (blockIdx.x == 0)
        return;
    const int off = bsum[blockIdx.x - 1];
    const int64_t base = blockIdx.x * static_cast<int64_t>(kScanTile);
    for (int k = threadIdx.x; k < kScanTile; k += kScanThreads)
        if (base + k < n)
            a[base + k] += off;
}

__global__ void __launch_bounds__(256) copy_kernel(int *__restrict__ dst, const int *__restrict__ srcp, int64_t n)
{
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        dst[i] = srcp[i];
}

__global__ void __launch_bounds__(256) scatter_kernel(int64_t E, const int *__restrict__ src, int *__restrict__ cursor,
                                                      int *__restrict__ perm)
{
    for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < E;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int pos = atomicAdd(&cursor[src[e]], 1);
        perm[pos] = static_cast<int>(e);
    }
}

// Sort each source segment of perm by edge id. scratch (E ints) backs the
// rank-by-counting path for segments longer than kSortCap.
__global__ void __launch_bounds__(256) seg_sort_kernel(int n_src, const int *__restrict__ src_ptr, int *__restrict__ perm,
                                                       int *__restrict__ scratch)
{
    __shared__ int buf[kSortCap];
    const int j = blockIdx.x;
    if (j >= n_src)
        return;
    const int s = src_ptr[j], len = src_ptr[j + 1] - s;
    if (len <= 1)
        return;
    if (len <= kSortCap) {
        int n2 = 1;
        while (n2 < len)
            n2 <<= 1;
        for (int i = threadIdx.x; i < n2; i += blockDim.x)
            buf[i] = i < len ? perm[s + i] : INT_MAX;
        __syncthreads();
        for (int k = 2; k <= n2; k <<= 1) {
            for (int jj = k >> 1; jj > 0; jj >>= 1) {
                for (int i = threadIdx.x; i < n2; i += blockDim.x) {
                    const int ixj = i ^ jj;
                    if (ixj > i) {
                        const bool up = (i & k) == 0;
                        const int a = buf[i], b = buf[ixj];
                        if ((a > b) == up) {
                            buf[i] = b;
                            buf[ixj] = a;
                        }
                    }
                }
                __syncthreads();
            }
        }
        for (int i = threadIdx.x; i < len; i += blockDim.x)
            perm[s + i] = buf[i];
    } else {
        for (int i = threadIdx.x; i < len; i += blockDim.x)
            scratch[s + i] = perm[s + i];
        __syncthreads();
        for (int i = threadIdx.x; i < len; i += blockDim.x) {
            const int v = scratch[s + i];
            int r = 0;
            for (int k = 0; k < len; ++k)
                r += scratch[s + k] < v;
            perm[s + r] = v;
        }
    }
}

__global__ void __launch_bounds__(256) dst_lookup_kernel(int64_t E, int n_dst, const int *__restrict__ row_ptr,
                                                         const int *__restrict__ perm, int *__restrict__ perm_dst)
{
    for (int64_t k = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; k < E;
         k += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int e = perm[k];
        // first index with row_ptr[idx] > e, minus one
        int lo = 0, hi = n_dst + 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (row_ptr[mid] > e)
                hi = mid;
            else
                lo = mid + 1;
        }
        perm_dst[k] = lo - 1;
    }
}

// Counts violations of: row_ptr[0] == 0, row_ptr non-decreasing,
// row_ptr[n_dst] == E, 0 <= src[e] < n_src (src may be null: not checked).
__global__ void __launch_bounds__(256) validate_kernel(int n_dst, int n_src, int64_t E, const int *__restrict__ row_ptr,
                                                       const int *__restrict__ src, int *__restrict__ bad)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t t0 = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
    int nbad = 0;
    for (int64_t i = t0; i < n_dst; i += stride)
        nbad += row_ptr[i] > row_ptr[i + 1];
    if (src)
        for (int64_t e = t0; e < E; e += stride)
            nbad += (src[e] < 0 || src[e] >= n_src);
    if (t0 == 0)
        nbad += (row_ptr[0] != 0) + (static_cast<int64_t>(row_ptr[n_dst]) != E);
    if (nbad)
        atomicAdd(bad, nbad);
}

static unsigned grid_for(int64_t n)
{
    const int64_t b = (n + 255) / 256;
    return static_cast<unsigned>(b < 1 ? 1 : (b > 16384 ? 16384 : b));
}

int64_t scan_bsum_ints(int64_t n) { return (n + kScanTile - 1) / kScanTile + 1; }

template <int TAG>
static hipError_t fill_int(int *p, int64_t n, int v, hipStream_t stream)
{
    if (n > 0)
        hipLaunchKernelGGL(fill_kernel<TAG>, dim3(grid_for(n)), dim3(256), 0, stream, p, n, v);
    return hipGetLastError();
}

hipError_t launch_nl_fill_int(int *p, int64_t n, int v, hipStream_t stream)
{
    return fill_int<kTagNeighbors>(p, n, v, stream);
}

// ptr[1..n] hold counts; on return ptr[k] = the sum of counts 1..k, i.e.
// the offsets of a CSR when ptr[0] = 0 (ptr[0] is not touched). bsum holds
// scan_bsum_ints(n) ints.
template <int TAG>
static hipError_t counts_to_offsets(int *ptr, int64_t n, int *bsum, hipStream_t stream)
{
    if (n <= 0)
        return hipGetLastError();
    const int64_t ntile = (n + kScanTile - 1) / kScanTile;
    hipLaunchKernelGGL(scan_tiles_kernel<TAG>, dim3(static_cast<unsigned>(ntile)), dim3(kScanThreads), 0, stream,
                       ptr + 1, n, bsum);
    if (ntile > 1) {
        hipLaunchKernelGGL(scan_single_kernel<TAG>, dim3(1), dim3(kScanThreads), 0, stream, bsum, ntile);
        hipLaunchKernelGGL(add_offsets_kernel<TAG>, dim3(static_cast<unsigned>(ntile)), dim3(kScanThreads), 0,
                           stream, ptr + 1, n, bsum);
    }
    return hipGetLastError();
}

hipError_t launch_nl_counts_to_offsets(int *ptr, int64_t n, int *bsum, hipStream_t stream)
{
    return counts_to_offsets<kTagNeighbors>(ptr, n, bsum, stream);
}

size_t transpose_workspace_bytes(int n_src)
{
    const int64_t ntile = (static_cast<int64_t>(n_src) + kScanTile - 1) / kScanTile;
    return sizeof(int) * static_cast<size_t>(n_src + ntile + 64);
}

hipError_t launch_transpose(int n_dst, int n_src, int64_t E, const int *row_ptr, const int *src, int *src_ptr,
                            int *perm, int *perm_dst, void *ws, hipStream_t stream)
{
    int *cursor = static_cast<int *>(ws);
    const int64_t ntile = (static_cast<int64_t>(n_src) + kScanTile - 1) / kScanTile;
    int *bsum = cursor + n_src;
    hipError_t err = fill_int<kTagTranspose>(src_ptr, static_cast<int64_t>(n_src) + 1, 0, stream);
    if (err != hipSuccess)
        return err;
    if (E > 0)
        hipLaunchKernelGGL(hist_kernel, dim3(grid_for(E)), dim3(256), 0, stream, E, src, src_ptr + 1);
    if (n_src > 0) {
        err = counts_to_offsets<kTagTranspose>(src_ptr, n_src, bsum, stream);
        if (err != hipSuccess)
            return err;
        hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n_src)), dim3(256), 0, stream, cursor, src_ptr,
                           static_cast<int64_t>(n_src));
    }
    if (E > 0) {
        hipLaunchKernelGGL(scatter_kernel, dim3(grid_for(E)), dim3(256), 0, stream, E, src, cursor, perm);
        hipLaunchKernelGGL(seg_sort_kernel, dim3(static_cast<unsigned>(n_src)), dim3(256), 0, stream, n_src,
                           src_ptr, perm, perm_dst);
        hipLaunchKernelGGL(dst_lookup_kernel, dim3(grid_for(E)), dim3(256), 0, stream, E, n_dst, row_ptr, perm,
                           perm_dst);
    }
    return hipGetLastError();
}

// ------------------------------------------------------- ordered block sum
// out[t] (+)= sum over j < n of part[j * stride + t], t < total, in the order
// of j: level 1 sums runs of up to `per` consecutive blocks into tmp[g][t],
// level 2 adds the runs in order (a fixed order throughout: deterministic).
// Used for weight gradients that are sums over all nodes of per-node partials.
constexpr int kBlockSumRuns = 64;

__global__ void __launch_bounds__(256) block_sum_l1_kernel(int64_t n, int64_t stride, int total, int64_t per,
                                                          const float *__restrict__ part, float *__restrict__ tmp)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= total)
        return;
    const int64_t j0 = blockIdx.y * per, j1 = (j0 + per < n) ? j0 + per : n;
    float s = 0.f;
    for (int64_t j = j0; j < j1; ++j)
        s += part[j * stride + t];
    tmp[static_cast<int64_t>(blockIdx.y) * total + t] = s;
}

__global__ void __launch_bounds__(256) block_sum_l2_kernel(int runs, int total, const float *__restrict__ tmp,
                                                          float *__restrict__ out, int accumulate)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= total)
        return;
    float s = 0.f;
    for (int g = 0; g < runs; ++g)
        s += tmp[static_cast<int64_t>(g) * total + t];
    out[t] = accumulate ? out[t] + s : s;
}

size_t block_sum_tmp_floats(int total) { return static_cast<size_t>(kBlockSumRuns) * total; }

hipError_t launch_block_sum(int64_t n, int64_t stride, int total, const float *part, float *tmp, float *out,
                            bool accumulate, hipStream_t stream)
{
    if (total <= 0)
        return hipSuccess;
    const int64_t per = n > 0 ? (n + kBlockSumRuns - 1) / kBlockSumRuns : 1;
    const unsigned bx = static_cast<unsigned>((total + 255) / 256);
    hipLaunchKernelGGL(block_sum_l1_kernel, dim3(bx, kBlockSumRuns), dim3(256), 0, stream, n, stride, total, per, part,
                       tmp);
    hipLaunchKernelGGL(block_sum_l2_kernel, dim3(bx), dim3(256), 0, stream, kBlockSumRuns, total, tmp, out,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

// ---------------------------------------------------- no-allocation variant
// The transpose's workspace (the per-source cursors and the scan's tile
// totals) for callers that cannot allocate: a file-scope device array of
// fixed size, one copy per GPU, shared by every call on that GPU. The
// transpose writes every word it reads from it within the same call, so its
// contents need no clearing between calls; calls that overlap on one GPU
// race on it.
constexpr int kNoAllocSources = 1 << 20;
constexpr size_t kNoAllocInts =
    static_cast<size_t>(kNoAllocSources) + (kNoAllocSources + kScanTile - 1) / kScanTile + 64;
static __device__ __align__(256) int scratch[kNoAllocInts];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int *g_scratch[kMaxDevices];  // the device address of scratch, per device (set once)
}  // namespace

// The current device's copy of scratch, looked up once per device (in host
// code the array's name is not a device address).
static hipError_t scratch_of_current_device(int **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch[dev] = static_cast<int *>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

int transpose_noalloc_max_sources() { return kNoAllocSources; }

hipError_t launch_transpose_noalloc(int n_dst, int n_src, int64_t E, const int *row_ptr, const int *src,
                                    int *src_ptr, int *perm, int *perm_dst, hipStream_t stream)
{
    if (n_src < 0 || n_src > kNoAllocSources || transpose_workspace_bytes(n_src) > sizeof(int) * kNoAllocInts)
        return hipErrorInvalidValue;
    int *ws = nullptr;
    const hipError_t e = scratch_of_current_device(&ws);
    if (e != hipSuccess)
        return e;
    return launch_transpose(n_dst, n_src, E, row_ptr, src, src_ptr, perm, perm_dst, ws, stream);
}

hipError_t launch_validate(int n_dst, int n_src, int64_t E, const int *row_ptr, const int *src, int *bad,
                           hipStream_t stream)
{
    hipLaunchKernelGGL(validate_kernel, dim3(grid_for(E > n_dst ? E : n_dst)), dim3(256), 0, stream, n_dst, n_src, E,
                       row_ptr, src, bad);
    return hipGetLastError();
}

}  // namespace etp
