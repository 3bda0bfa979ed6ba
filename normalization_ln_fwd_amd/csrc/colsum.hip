// colsum.hip -- the backward's second stage (column sums of the per-workgroup
// partials plus the down-cast) and the amax reset.
#include "kernels.hpp"
#include "normfuse.h"

namespace nf {

static_assert(NORM_AMAX_WS_BYTES >= (AMAX_SUBGROUPS + 1) * AMAX_CELL_WORDS * sizeof(unsigned),
              "the amax workspace holds every arrival cell");

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

// Thread layouts of the column sums (columns per tile 4 * QUADS, SUB row
// subsets, RPT rows per subset loaded at once; SUB * RPT covers a slice in
// one pass, so every thread's loads are in flight together):
//  - slices of many partial rows (COLSUM_SPAN rows each): 64-column tiles;
//  - final sums of up to FEW_ROWS rows: 32-column tiles of 256 threads, e.g.
//    128 tiles per block at 4096 columns;
//  - final sums of up to COLSUM_ONE_LAUNCH rows: 32-column tiles of 512
//    threads.
// Measured on MI355X, the column sums of the 8192 x 4096 bf16 backward (256
// partial rows of dgamma and dbeta): 4.4 us per launch in a kernel trace
// when each thread walked its rows four loads at a time, 16 rows deep.
constexpr int SLICE_QUADS = 16, SLICE_SUB = 16, SLICE_RPT = COLSUM_SPAN / SLICE_SUB;
constexpr int FEW_QUADS = 8, FEW_SUB = 32, FEW_RPT = 8, FEW_ROWS = FEW_SUB * FEW_RPT;
constexpr int FINAL_QUADS = 8, FINAL_SUB = 64, FINAL_RPT = COLSUM_ONE_LAUNCH / FINAL_SUB;

template <int QUADS, int SUB, int RPT>
hipError_t launch_final(const float *src, int rows, int nb, int N, void *dgamma, void *dbeta,
                        void *dbias, int out_dtype, float divisor, hipStream_t s)
{
    const dim3 grid(unsigned((N + 4 * QUADS - 1) / (4 * QUADS)), 1, nb);
    const dim3 block(QUADS * SUB);
    if (out_dtype == 1)
        hipLaunchKernelGGL((colsum_kernel<true, true, QUADS, SUB, RPT>), grid, block, 0, s, src,
                           rows, N, rows, nullptr, dgamma, dbeta, dbias, divisor);
    else
        hipLaunchKernelGGL((colsum_kernel<true, false, QUADS, SUB, RPT>), grid, block, 0, s, src,
                           rows, N, rows, nullptr, dgamma, dbeta, dbias, divisor);
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
        hipLaunchKernelGGL((colsum_kernel<false, false, SLICE_QUADS, SLICE_SUB, SLICE_RPT>),
                           dim3(tiles, slices, nb), dim3(SLICE_QUADS * SLICE_SUB), 0, s, ws,
                           parts, N, COLSUM_SPAN, level2, nullptr, nullptr, nullptr, 1.f);
        if (hipError_t e = hipGetLastError())
            return e;
        src = level2;
        rows = slices;
    }
    if (rows <= FEW_ROWS)
        return launch_final<FEW_QUADS, FEW_SUB, FEW_RPT>(src, rows, nb, N, dgamma, dbeta, dbias,
                                                         out_dtype, divisor, s);
    return launch_final<FINAL_QUADS, FINAL_SUB, FINAL_RPT>(src, rows, nb, N, dgamma, dbeta,
                                                           dbias, out_dtype, divisor, s);
}

} // namespace nf
