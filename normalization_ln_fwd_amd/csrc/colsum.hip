// colsum.hip -- the backward's second stage (column sums of the per-workgroup
// partials plus the down-cast) and the amax reset.
#include "kernels.hpp"

namespace nf {

__global__ void __launch_bounds__(64) zero_u32_kernel(unsigned *p)
{
    if (threadIdx.x == 0)
        *p = 0u;
}

hipError_t launch_zero_u32(unsigned *p, hipStream_t s)
{
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_colsum(const float *ws, int parts, int nb, int N, void *dgamma, void *dbeta,
                         void *dbias, int out_dtype, float divisor, float *level2, hipStream_t s)
{
    if (dgamma == nullptr && dbeta == nullptr && dbias == nullptr)
        return hipSuccess;
    const unsigned tiles = unsigned((N + COLSUM_COLS - 1) / COLSUM_COLS);
    const dim3 block(COLSUM_QUADS * COLSUM_SUB);
    const float *src = ws;
    int rows = parts;
    const int slices = colsum_slices(parts);
    if (slices > 1) {
        hipLaunchKernelGGL((colsum_kernel<false, false>), dim3(tiles, slices, nb), block, 0, s,
                           ws, parts, N, COLSUM_SPAN, level2, nullptr, nullptr, nullptr, 1.f);
        if (hipError_t e = hipGetLastError())
            return e;
        src = level2;
        rows = slices;
    }
    if (out_dtype == 1)
        hipLaunchKernelGGL((colsum_kernel<true, true>), dim3(tiles, 1, nb), block, 0, s, src,
                           rows, N, rows, nullptr, dgamma, dbeta, dbias, divisor);
    else
        hipLaunchKernelGGL((colsum_kernel<true, false>), dim3(tiles, 1, nb), block, 0, s, src,
                           rows, N, rows, nullptr, dgamma, dbeta, dbias, divisor);
    return hipGetLastError();
}

} // namespace nf
