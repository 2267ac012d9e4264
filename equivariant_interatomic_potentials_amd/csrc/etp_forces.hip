// etp_forces.hip -- forces on the atoms from the per-edge gradients of the
// energy with respect to the bond vectors (energy and forces from one model:
// "How does FlashCart make equivariant interatomic potentials faster and
// more accurate?", section on the SPICE-MACE-OFF model).
//
// With vec_e = pos[src_e] - pos[dst_e] and gr_e = dE/dvec_e:
//   F[k] = -dE/dpos[k] = sum_{e in in(k)} gr_e - sum_{e in out(k)} gr_e.
//
// Mapping (gfx950, wave64): one wave per atom; lane t takes the atom's
// in-edges t, t + 64, ... (the destination-sorted CSR) and then its
// out-edges in the same way (the stable transpose), three running sums per
// lane, then a fixed-order DPP sum; lane 63 writes the force. No atomics, so
// the result does not depend on scheduling.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "etp_device.hpp"

namespace etp {

__global__ void __launch_bounds__(256) forces_kernel(const int n_dst, const int n_src, const int n,
                                                     const int *__restrict__ row_ptr, const int *__restrict__ src_ptr,
                                                     const int *__restrict__ perm, const float *__restrict__ gr,
                                                     float *__restrict__ F, const int accumulate)
{
    const int lane = threadIdx.x & 63;
    const int k = blockIdx.x * 4 + wave_id();
    if (k >= n)
        return;
    float f0 = 0.f, f1 = 0.f, f2 = 0.f;
    if (k < n_dst) {
        for (int e = row_ptr[k] + lane; e < row_ptr[k + 1]; e += 64) {
            f0 += gr[3 * static_cast<int64_t>(e)];
            f1 += gr[3 * static_cast<int64_t>(e) + 1];
            f2 += gr[3 * static_cast<int64_t>(e) + 2];
        }
    }
    if (k < n_src) {
        for (int q = src_ptr[k] + lane; q < src_ptr[k + 1]; q += 64) {
            const int64_t e = perm[q];
            f0 -= gr[3 * e];
            f1 -= gr[3 * e + 1];
            f2 -= gr[3 * e + 2];
        }
    }
    f0 = wave_sum_to_lane63(f0);
    f1 = wave_sum_to_lane63(f1);
    f2 = wave_sum_to_lane63(f2);
    if (lane == 63) {
        float *fk = F + 3 * static_cast<int64_t>(k);
        if (accumulate) {
            f0 += fk[0];
            f1 += fk[1];
            f2 += fk[2];
        }
        fk[0] = f0;
        fk[1] = f1;
        fk[2] = f2;
    }
}

hipError_t launch_forces(int n_dst, int n_src, const int *row_ptr, const int *src_ptr, const int *perm,
                         const float *gr, float *F, bool accumulate, hipStream_t stream)
{
    const int n = n_dst > n_src ? n_dst : n_src;
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(forces_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, n_dst, n_src, n, row_ptr, src_ptr,
                       perm, gr, F, accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace etp
