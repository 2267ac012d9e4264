// etp_sh.hip -- standalone real spherical harmonics of bond vectors (the SH
// that the convolution kernels evaluate in registers), with the optional
// gradient with respect to the unnormalised vector (the force path's
// Jacobian).
#include "etp_conv_common.hpp"

namespace etp {

template <int L>
__global__ void __launch_bounds__(256) sh_kernel(const int64_t n, const float *__restrict__ vec,
                                                 float *__restrict__ Y, float *__restrict__ dY)
{
    constexpr int D = (L + 1) * (L + 1);
    for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const float rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
        float *yp = Y + e * D;
        if (dY == nullptr) {
            float v[D];
            sh_value<L>(rx, ry, rz, v);
            static_range<0, D>([&](auto b) { yp[b] = v[b]; });
        } else {
            D3 v[D];
            sh_grad<L>(rx, ry, rz, v);
            float *dp = dY + e * 3 * D;
            static_range<0, D>([&](auto b) {
                yp[b] = v[b].v;
                dp[b] = v[b].g0;
                dp[D + b] = v[b].g1;
                dp[2 * D + b] = v[b].g2;
            });
        }
    }
}

hipError_t launch_sh(int L, int64_t n, const float *vec, float *Y, float *dY, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const int64_t want = (n + 255) / 256;
    const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
    switch (L) {
    case 0: hipLaunchKernelGGL(sh_kernel<0>, dim3(blocks), dim3(256), 0, stream, n, vec, Y, dY); break;
    case 1: hipLaunchKernelGGL(sh_kernel<1>, dim3(blocks), dim3(256), 0, stream, n, vec, Y, dY); break;
    case 2: hipLaunchKernelGGL(sh_kernel<2>, dim3(blocks), dim3(256), 0, stream, n, vec, Y, dY); break;
    case 3: hipLaunchKernelGGL(sh_kernel<3>, dim3(blocks), dim3(256), 0, stream, n, vec, Y, dY); break;
    case 4: hipLaunchKernelGGL(sh_kernel<4>, dim3(blocks), dim3(256), 0, stream, n, vec, Y, dY); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace etp
