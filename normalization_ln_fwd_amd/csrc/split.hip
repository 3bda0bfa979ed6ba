// split.hip -- the backward with rows split along N (bwd_split_kernel):
// instantiations for the 16-byte paths and the two-pass launch.
#include "kernels.hpp"

namespace nf {

int split_chunk_cols(int32_t dtype) { return dtype == 0 ? split_cols<float, 4>() : split_cols<bf16, 8>(); }

template <typename T, int VEC, bool RMS, bool DB>
hipError_t split_passes(const BwdArgs &a, int blocks, hipStream_t s)
{
    const dim3 grid(unsigned(a.chunks), unsigned(blocks));
    const dim3 block(64 * SPLIT_ROWS_PER_GROUP);
    hipLaunchKernelGGL((bwd_split_kernel<T, VEC, RMS, DB, 0>), grid, block, 0, s, a);
    if (hipError_t e = hipGetLastError())
        return e;
    hipLaunchKernelGGL((bwd_split_kernel<T, VEC, RMS, DB, 1>), grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_split(const BwdArgs &a, int32_t dtype, bool rms, bool dbias, int blocks,
                            hipStream_t s)
{
    if (dtype == 0) {
        if (rms)
            return dbias ? split_passes<float, 4, true, true>(a, blocks, s)
                         : split_passes<float, 4, true, false>(a, blocks, s);
        return dbias ? split_passes<float, 4, false, true>(a, blocks, s)
                     : split_passes<float, 4, false, false>(a, blocks, s);
    }
    if (rms)
        return dbias ? split_passes<bf16, 8, true, true>(a, blocks, s)
                     : split_passes<bf16, 8, true, false>(a, blocks, s);
    return dbias ? split_passes<bf16, 8, false, true>(a, blocks, s)
                 : split_passes<bf16, 8, false, false>(a, blocks, s);
}

} // namespace nf
