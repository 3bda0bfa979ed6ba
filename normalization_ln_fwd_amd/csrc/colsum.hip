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

hipError_t launch_colsum(const float *ws, int grid_parts, int N, void *dgamma, void *dbeta,
                         int out_dtype, hipStream_t s)
{
    if (dgamma == nullptr && dbeta == nullptr)
        return hipSuccess;
    const dim3 grid((N + COLSUM_COLS - 1) / COLSUM_COLS, 2);
    const dim3 block(COLSUM_COLS * COLSUM_SLICES);
    if (out_dtype == 1)
        hipLaunchKernelGGL(colsum_kernel<true>, grid, block, 0, s, ws, grid_parts, N, dgamma, dbeta);
    else
        hipLaunchKernelGGL(colsum_kernel<false>, grid, block, 0, s, ws, grid_parts, N, dgamma, dbeta);
    return hipGetLastError();
}

} // namespace nf
