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

// Thread layouts of the column sums: the slices of many partial rows take
// 64-column tiles of 16 row subsets; the final sums take 32-column tiles of
// 128 subsets, so that a few hundred rows of a wide N spread over all CUs
// with every thread's loads issued at once.  Final sums of at most
// FEW_ROWS rows take 64-column tiles of 16 subsets instead: an eighth of
// the waves, which at these counts would mostly idle and still cost their
// launch (measured on MI355X, whole backward calls: 1 x 16384 bf16 11.7 ->
// 8.8 us, 1024 x 16384 38.5 -> 35.7 us).
constexpr int SLICE_QUADS = 16, SLICE_SUB = 16;
constexpr int FINAL_QUADS = 8, FINAL_SUB = 128;
constexpr int FEW_QUADS = 16, FEW_SUB = 16, FEW_ROWS = 256;

template <int QUADS, int SUB>
hipError_t launch_final(const float *src, int rows, int nb, int N, void *dgamma, void *dbeta,
                        void *dbias, int out_dtype, float divisor, hipStream_t s)
{
    const dim3 grid(unsigned((N + 4 * QUADS - 1) / (4 * QUADS)), 1, nb);
    const dim3 block(QUADS * SUB);
    if (out_dtype == 1)
        hipLaunchKernelGGL((colsum_kernel<true, true, QUADS, SUB>), grid, block, 0, s, src, rows, N,
                           rows, nullptr, dgamma, dbeta, dbias, divisor);
    else
        hipLaunchKernelGGL((colsum_kernel<true, false, QUADS, SUB>), grid, block, 0, s, src, rows,
                           N, rows, nullptr, dgamma, dbeta, dbias, divisor);
    return hipGetLastError();
}

hipError_t launch_colsum(const float *ws, int parts, int nb, int N, void *dgamma, void *dbeta,
                         void *dbias, int out_dtype, float divisor, float *level2, hipStream_t s)
{
    if (dgamma == nullptr && dbeta == nullptr && dbias == nullptr)
        return hipSuccess;
    const float *src = ws;
    int rows = parts;
    const int slices = colsum_slices(parts);
    if (slices > 1) {
        const unsigned tiles = unsigned((N + 4 * SLICE_QUADS - 1) / (4 * SLICE_QUADS));
        hipLaunchKernelGGL((colsum_kernel<false, false, SLICE_QUADS, SLICE_SUB>),
                           dim3(tiles, slices, nb), dim3(SLICE_QUADS * SLICE_SUB), 0, s, ws,
                           parts, N, COLSUM_SPAN, level2, nullptr, nullptr, nullptr, 1.f);
        if (hipError_t e = hipGetLastError())
            return e;
        src = level2;
        rows = slices;
    }
    if (rows <= FEW_ROWS)
        return launch_final<FEW_QUADS, FEW_SUB>(src, rows, nb, N, dgamma, dbeta, dbias, out_dtype,
                                                divisor, s);
    return launch_final<FINAL_QUADS, FINAL_SUB>(src, rows, nb, N, dgamma, dbeta, dbias, out_dtype,
                                                divisor, s);
}

} // namespace nf
